"""Benchmark of the TurboQuant hot path on one MI355X.

Workload: the Llama-3.1-8B-shaped decode layer (32 query heads, 8 KV heads,
head_dim 128, batch 1, 32768 cached tokens, bf16 K/V N(0, 1) with 4 outlier
channels per KV head scaled by 10, b = 4, logits for one new token).  One
step runs that layer's hot path for L = 32 independent layer caches (as in a
32-layer model, so the 704 MB of packed keys and logits per step are well
beyond the 256 MB Infinity Cache): quantize each layer's new-token K and V
into its packed cache and rotate/project each layer's 32 query heads (one
launch: tq_decode_step_prepare), then stream all cached keys of every layer
into attention logits (one launch).

Outside the timed steps: a cache-fill leg times tq_quantize_kv on all K and V
of the 32 layers (quantize vectors/s), and the CPU oracle is timed on a
bounded sample of the same decode work (cpu_baseline).

Other workloads (each prints its own JSON line; the default is the one above):
  --workload long     8 KV heads x 131072 tokens, bf16 N(0,1), b in {2,3,4}:
                      quantize K+V and 32 x 131072 logits per b (MALL-cold
                      reps: a 1 GiB buffer is written before each rep)
  --workload batched  16 ragged sequences (4096..8192 tokens), b = 3: quantize
                      a 512-token chunk per sequence, then logits for one
                      query of 32 heads per sequence
  --workload attn_out the value side of the Llama-shaped decode layer over 32
                      layer caches: tq_attn_output (weights from a softmax of
                      seeded logits) over all packed values of every layer
  --workload decode_fused  fused decode attention (tq_attn_decode: logits,
                      softmax, value sums) over the same 32 layer caches
  --workload search   1e6 unit vectors at d = 1536 or 200 (--search-d), b in
                      {2, 4} (--bits): quantize the database, then score 1000
                      queries against all of it and keep the top 10
  --workload stream_ceiling  the references the kernels are measured against
                      (libtq_ceiling.so): a plain stream with the logit
                      kernel's read/write mix over the default workload's
                      8.39 M records, a 1 GiB device copy, int8 / bf16
                      matrix-core loops, and MFMA / vector-ALU co-issue

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "long", "batched", "search", "attn_out", "decode_fused",
                             "split", "dequant", "stream_ceiling"])
    ap.add_argument("--search-d", type=int, default=1536)
    ap.add_argument("--bits", type=int, default=0, help="search / long: one b (default all)")
    ap.add_argument("--mse", action="store_true",
                    help="long / search / attn_out / decode_fused: MSE-only records (b code "
                         "bits, no QJL stage; b = 1..3)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device copy of this size (for scaling HBM "
                         "byte counters)")
    return ap.parse_args()


PROFILE_LOGITS = os.path.join(ROOT, "profiles", "attn_logits_llama8b_decode_32layers.md")
PROFILE_DEQUANT = os.path.join(ROOT, "profiles", "dequantize_llama_layer.md")
# sources of the logit kernel (hashed together, in this order)
LOGIT_SOURCES = [os.path.join(ROOT, "kv_cache_vector_pi_amd", "csrc", f)
                 for f in ("tq_logits.hip", "tq_dev.h")]


DEQUANT_SOURCES = [os.path.join(ROOT, "kv_cache_vector_pi_amd", "csrc", "tq_search.hip")]


def profiled_traffic(profile, sources):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel sources have changed since the counters were taken."""
    import hashlib
    try:
        text = open(profile).read()
        h = hashlib.sha256()
        for f in sources:
            h.update(open(f, "rb").read())
        src = h.hexdigest()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if ":" in line and line.strip().startswith("- `"):
            k, v = line.strip()[3:].split("`", 1)[0], line.split(":", 1)[1]
            parts = v.split("`")
            vals[k] = parts[1] if len(parts) >= 3 else v.strip()
    if vals.get("kernel_source_sha256") != src:
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the hot path has no multi-GPU leg.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_vector_pi_amd as tq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.mse and args.workload in ("decode", "batched"):
        print("--mse applies to the long, search, attn_out and decode_fused workloads",
              file=sys.stderr)
        sys.exit(2)
    if args.workload != "decode":
        out = {"long": run_long, "batched": run_batched, "search": run_search,
               "attn_out": run_attn_out, "decode_fused": run_decode_fused,
               "split": run_split, "dequant": run_dequant,
               "stream_ceiling": run_stream_ceiling}[args.workload](args)
        print(json.dumps(out), flush=True)
        return
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
        # one launch: quantize the new K and V token of each (kv head, layer)
        # ("head" = (h, l) pair) and prepare the 32 layers' queries
        tq.tq_decode_step_prepare(ctx, newK.view(N_KV * L, 1, D), newV.view(N_KV * L, 1, D),
                                  k_planes, k_norms, v_planes, v_norms, q_all, L, N_Q, N_Q * D,
                                  N_KV, ws, dst_stride_head=N_TOK, dst_token0=N_TOK - 1)
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
        cpu = cpu_oracle_baseline(args, k_planes, k_norms, newK, newV, q_all, L, scale)

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
        "roofline": {"bound": "hbm", "kernel": "attn_logits_res_kernel<4,false,4,0,false>",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": profiled_traffic(PROFILE_LOGITS, LOGIT_SOURCES),
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


def host_cpu():
    """(logical CPUs, CPU model) of this host."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return os.cpu_count(), model


def cpu_oracle_baseline(args, k_planes, k_norms, newK, newV, q_all, L, scale):
    """The fp64 oracle on a bounded sample of the decode step: per layer, the
    new token's K and V of every KV head quantized, and the 32 heads' logits
    over that layer's 32768 cached keys -- the records the GPU wrote (layer 0's
    caches, copied to the host outside the timed region)."""
    import numpy as np
    import oracle
    _, _, opi, os_ = oracle.make_rotation(D, 0)
    oc = oracle.lloyd_max(D, B - 1)[0].astype(np.float32)
    G = N_Q // N_KV
    kp = k_planes.view(N_KV, L, N_TOK, -1)[:, 0].cpu().numpy().view(np.uint32)
    kn = k_norms.view(N_KV, L, N_TOK, 2)[:, 0].cpu().numpy().view(np.uint16)
    q0 = q_all[0].double().cpu().numpy()
    newk = newK[:, 0].double().cpu().numpy()        # [8][128]: layer 0's new token
    newv = newV[:, 0].double().cpu().numpy()
    done_logits, t_cpu = 0, 0.0
    while t_cpu < args.cpu_seconds or done_logits == 0:
        c0 = time.perf_counter()
        oracle.quantize(D, B, opi, os_, oc, newk)
        oracle.quantize(D, B, opi, os_, oc, newv)
        for h in range(N_KV):
            oracle.estimate(D, B, opi, os_, oc, q0[G * h:G * (h + 1)], kp[h], kn[h], scale=scale)
        t_cpu += time.perf_counter() - c0
        done_logits += N_Q * N_TOK
    nproc, model = host_cpu()
    return {"value": done_logits / t_cpu, "unit": "logits/s", "cores": oracle.num_threads(),
            "kind": "oracle", "nproc": nproc, "cpu_model": model,
            "sample": f"{done_logits // (N_Q * N_TOK)} decode layer(s) of the same shape: "
                      f"the new K and V token of 8 KV heads quantized, then 32 q heads x "
                      f"32768 logits from the GPU-written packed keys of layer 0, "
                      f"{t_cpu:.1f} s of fp64 oracle work"}


# ---- other workloads ---------------------------------------------------------
def _timed(fn, reps, stream, flush=None):
    """(mean, median) ms of fn() over reps with HIP events on `stream`;
    flush() (untimed) runs before each rep."""
    import torch
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    return sum(ts) / len(ts), ts[len(ts) // 2]


def _common(args, d, b, seed=0):
    import kv_cache_vector_pi_amd as tq
    pi, s = tq.tq_make_rotation(d, seed)
    if getattr(args, "mse", False):
        cent, _, _ = tq.tq_lloyd_max(d, b)
        return tq.TqContext(d, b, pi, None, cent)
    cent, _, _ = tq.tq_lloyd_max(d, b - 1)
    return tq.TqContext(d, b, pi, s, cent)


def _bits(args, two_stage, mse):
    if args.bits:
        return [args.bits]
    return mse if args.mse else two_stage


def _line(args, metric, value, unit, workload, extra):
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "data": "synthetic (seeded)", "config": workload}
    out.update(extra)
    if getattr(args, "mse", False):
        out["config"] = dict(out["config"], records="MSE-only: b code bits, no QJL stage")
    return out


def run_stream_ceiling(args):
    """Ceilings: the logit stream's byte mix as a plain stream, a plain copy,
    and matrix-core loops (include/tq_ceiling.h)."""
    import ctypes
    import torch
    import kv_cache_vector_pi_amd as tq
    dev = "cuda"
    lib = ctypes.CDLL(os.path.join(os.path.dirname(tq.LIB_PATH), "libtq_ceiling.so"))
    P = ctypes.c_void_p
    lib.tq_ceiling_logit_mix.argtypes = [P, P, ctypes.c_int64, P, ctypes.c_int64, P]
    lib.tq_ceiling_copy.argtypes = [P, P, ctypes.c_int64, P]
    lib.tq_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    stream = torch.cuda.current_stream()
    sp = P(stream.cuda_stream)
    reps = max(5, min(args.steps, 50))

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"ceiling kernel failed: hipError {rc}")

    # the default workload's logit launch: 32 layers x 8 KV heads x 32768
    # records of 64 + 4 bytes in, 4 logits (16 bytes) out per record
    n = LAYERS * N_KV * N_TOK
    planes = torch.randint(-2**31, 2**31 - 1, (n, 16), dtype=torch.int32, device=dev)
    norms = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device=dev)
    out = torch.empty((4, n), dtype=torch.float32, device=dev)
    mix = lambda: ok(lib.tq_ceiling_logit_mix(P(planes.data_ptr()), P(norms.data_ptr()), n,
                                              P(out.data_ptr()), n, sp))
    for _ in range(args.warmup):
        mix()
    mix_ms, mix_med = _timed(mix, reps, stream)
    mix_bytes = n * (64 + 4 + 16)
    # the same bytes in one-shot workgroups of 128 / 512 records
    lib.tq_ceiling_logit_mix_blocks.argtypes = [P, P, ctypes.c_int64, P, ctypes.c_int64,
                                                ctypes.c_int, P]
    mixb = {}
    for per in (128, 512):
        fn = lambda p=per: ok(lib.tq_ceiling_logit_mix_blocks(
            P(planes.data_ptr()), P(norms.data_ptr()), n, P(out.data_ptr()), n, p, sp))
        for _ in range(args.warmup):
            fn()
        ms, med = _timed(fn, reps, stream)
        gbs = mix_bytes / (ms * 1e-3) / 1e9
        mixb[str(per)] = {"ms_mean": ms, "ms_median": med, "GB_per_s": gbs,
                          "frac": gbs / HBM_PEAK_GBS}
    del planes, norms, out
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    cp = lambda: ok(lib.tq_ceiling_copy(P(src.data_ptr()), P(dst.data_ptr()), nb, sp))
    for _ in range(args.warmup):
        cp()
    cp_ms, cp_med = _timed(cp, reps, stream)
    del src, dst
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 8 * n_cu, 2000
    sink = torch.empty(256 * blocks, dtype=torch.float32, device=dev)
    mf = {}
    for kind, name, ops in ((0, "i8_16x16x64", 2 * 16 * 16 * 64), (1, "bf16_32x32x16",
                                                                   2 * 32 * 32 * 16)):
        fn = lambda k=kind: ok(lib.tq_ceiling_mfma(k, blocks, iters, P(sink.data_ptr()), sp))
        for _ in range(2):
            fn()
        ms, _ = _timed(fn, 5, stream)
        mf[name] = blocks * 4 * iters * 8 * ops / (ms * 1e-3) / 1e12
    lib.tq_ceiling_overlap.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       P, P]
    ov = {}
    osink = torch.empty(512 * n_cu, dtype=torch.float32, device=dev)
    for kind, name in ((0, "fma"), (1, "compare_select")):
        t = []
        for mode in (0, 1, 2):
            fn = lambda m=mode, k=kind: ok(lib.tq_ceiling_overlap(m, k, n_cu, 2000,
                                                                  P(osink.data_ptr()), sp))
            fn()
            t.append(_timed(fn, 5, stream)[0])
        ov[name] = {"mfma_ms": t[0], "valu_ms": t[1], "both_ms": t[2],
                    "both_over_max": t[2] / max(t[0], t[1]), "both_over_sum": t[2] / (t[0] + t[1])}
    mix_gbs = mix_bytes / (mix_ms * 1e-3) / 1e9
    best_gbs = max([mix_gbs] + [v["GB_per_s"] for v in mixb.values()])
    return _line(args, "plain-stream ceiling with the logit kernel's byte mix", best_gbs, "GB/s",
                 {"workload": "stream ceiling: 8,388,608 records (64 B planes + 4 B norm read, "
                              "4 x 4 B written each) as a plain stream (the stream kernel's "
                              "tiling; one-shot workgroups of 128 / 512 records; value: the "
                              "fastest); 1 GiB copy; matrix-core loops of 8 workgroups x 4 "
                              "waves per CU"},
                 {"dtype": "u32 stream", "peak_GB_per_s": HBM_PEAK_GBS,
                  "logit_mix": {"ms_mean": mix_ms, "ms_median": mix_med, "GB_per_s": mix_gbs,
                                "frac": mix_gbs / HBM_PEAK_GBS, "bytes": mix_bytes},
                  "logit_mix_oneshot_blocks": mixb,
                  "copy_1GiB": {"ms_mean": cp_ms, "ms_median": cp_med,
                                "GB_per_s": 2 * nb / (cp_ms * 1e-3) / 1e9,
                                "frac": 2 * nb / (cp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
                  "mfma_TOPS": mf,
                  "mfma_valu_overlap": ov,
                  "mfma_peak_TOPS": {"i8_16x16x64": 5000.0, "bf16_32x32x16": 2500.0}})


def run_dequant(args):
    """tq_dequantize over one Llama-shaped layer's keys (8 KV heads x 32768
    tokens, d = 128, b = 4: 262,144 records to fp32 vectors), and the tiny
    configuration (1024 keys, d = 128, b = 3): its dequantize, quantize and
    16 x 1024 logits.  Calls back to back between two events on the launch
    stream."""
    import torch
    import kv_cache_vector_pi_amd as tq
    import workloads
    dev, d = "cuda", 128
    stream = torch.cuda.current_stream()
    reps = max(10, min(args.steps, 50))
    mse = getattr(args, "mse", False)
    res = {}
    for name, b, x in (("llama_layer", 3 if mse else 4, workloads.llama(dev, seed=0)["K"]),
                       ("tiny", 2 if mse else 3, workloads.tiny(dev)["K"])):
        x = x.reshape(-1, d).contiguous()
        n = x.shape[0]
        ctx = _common(args, d, b)
        planes, norms = tq.alloc_records(n, d, b, dev)
        tq.tq_quantize_kv(ctx, x, planes, norms)
        out = torch.empty((n, d), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            tq.tq_dequantize(ctx, planes, norms, n, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            tq.tq_dequantize(ctx, planes, norms, n, out)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        rb = b * d // 8 + 4
        alg_bytes = n * (rb + 4 * d)                 # packed record in, fp32 vector out
        alg_flops = n * 4 * d * d                    # Pi^T c[idx] and S^T s: 2 d^2 each
        # the kernel tq_dequantize picks: the register-resident d = 128 form
        # from 64 records per compute unit, else the general decoded GEMM
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        kern = (f"dequant128_kernel<{b},{'true' if mse else 'false'}>" if n >= 64 * n_cu
                else f"decoded_gemm_kernel<{b},{'true' if mse else 'false'},1>")
        res[name] = {"n": n, "b": b, "kernel": kern, "ms_per_call": ms,
                     "vec_per_s": n / (ms * 1e-3),
                     "GB_per_s": alg_bytes / (ms * 1e-3) / 1e9,
                     "TFLOP_per_s": alg_flops / (ms * 1e-3) / 1e12}
        if name == "tiny":
            # the rest of the tiny configuration: quantize the 1024 keys, and the
            # 16 x 1024 logits of its queries (one KV head, G = 16)
            q = workloads.tiny(dev)["Q"]
            ss = torch.zeros(1, dtype=torch.int64, device=dev)
            sl = torch.full((1,), n, dtype=torch.int32, device=dev)
            lg = torch.empty((16, n), dtype=torch.float32, device=dev)
            ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, 1, 16, 1), dev)

            def step_q():
                tq.tq_quantize_kv(ctx, x, planes, norms)

            def step_l():
                tq.tq_attn_logits(ctx, q, 1, 16, 16 * d, planes, norms, 1, n, ss, sl, n,
                                  1.0 / math.sqrt(d), lg, n, ws)
            for fn, key in ((step_q, "quantize_ms_per_call"), (step_l, "logits_ms_per_call")):
                for _ in range(args.warmup):
                    fn()
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(reps):
                    fn()
                e1.record(stream)
                e1.synchronize()
                res[name][key] = e0.elapsed_time(e1) / reps
        del ctx
    big = res["llama_layer"]
    return _line(args, "dequantize: vectors/s from packed records", big["vec_per_s"], "vectors/s",
                 {"workload": "dequantize one Llama-shaped layer's keys (8 KV heads x 32768 tokens, "
                              "d=128, b=%d) to fp32; tiny: 1024 keys, b=%d" %
                              (big["b"], res["tiny"]["b"])},
                 {"dtype": "fp16-mfma/fp32", "per_config": res,
                  "roofline": {"bound": "hbm", "kernel": big["kernel"],
                               "achieved": big["GB_per_s"], "peak": 8000.0, "unit": "GB/s",
                               "frac": big["GB_per_s"] / 8000.0,
                               "traffic": profiled_traffic(PROFILE_DEQUANT, DEQUANT_SOURCES),
                               "mfma_TFLOP_per_s_algorithmic": big["TFLOP_per_s"],
                               "mfma_frac_algorithmic": big["TFLOP_per_s"] / 2500.0}})


def run_split(args):
    """Fractional bit widths (two instances over a channel split: channels
    0..63 at b_hi bits, 64..127 at b_lo) on the Llama-shaped decode layer of
    the default workload: quantize the 32 layer caches' keys, then the logits
    of 32 layers x 32 heads against them, at 2.5 (3 + 2) and 3.5 (4 + 3) bits."""
    import torch
    import kv_cache_vector_pi_amd as tq
    import workloads
    dev = "cuda"
    stream = torch.cuda.current_stream()
    L, DH = args.layers, D // 2
    n_rec = N_KV * L * N_TOK
    Kx = torch.empty((N_KV, L * N_TOK, D), dtype=torch.bfloat16, device=dev)
    for l in range(L):
        Kx[:, l * N_TOK:(l + 1) * N_TOK] = workloads.llama(dev, seed=l, n_tok=N_TOK)["K"]
    torch.cuda.synchronize()
    q_all = torch.stack([workloads.normal((N_Q, D), l, workloads.STREAM_Q, dev)
                         for l in range(L)])
    seq_start = torch.arange(L, dtype=torch.int64, device=dev) * N_TOK
    seq_len = torch.full((L,), N_TOK, dtype=torch.int32, device=dev)
    logits = torch.empty((N_Q, L * N_TOK), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)
    reps = max(10, min(args.steps, 50))
    # attention weights for the value side (the packed keys stand in for
    # values: same record format and size)
    g = workloads.gen(0, workloads.STREAM_Q, dev)
    pw = torch.softmax(torch.randn((N_Q, L * N_TOK), generator=g, device=dev).view(N_Q, L, N_TOK),
                       dim=2).view(N_Q, L * N_TOK).contiguous()
    out = torch.empty((L, N_Q, D), device=dev)

    def inst(b, seed):
        pi, s = tq.tq_make_rotation(DH, seed)
        cent, _, _ = tq.tq_lloyd_max(DH, b - 1)
        return tq.TqContext(DH, b, pi, s, cent)

    def events(fn, n, before=None):
        # before(): launched ahead of the start event, so that fn's launch
        # queues behind it and the host-side launch time stays outside
        ts = []
        for _ in range(n):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            if before is not None:
                before()
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return sum(ts) / len(ts), sorted(ts)[len(ts) // 2]

    res = {}
    for bh, bl in ((3, 2), (4, 3)):
        hi, lo = inst(bh, 1), inst(bl, 2)
        hp = torch.empty((n_rec, tq.tq_record_words(DH, bh)), dtype=torch.int32, device=dev)
        lp = torch.empty((n_rec, tq.tq_record_words(DH, bl)), dtype=torch.int32, device=dev)
        hn = torch.empty((n_rec, 2), dtype=torch.int16, device=dev)
        ln = torch.empty_like(hn)
        ws = tq.workspace(tq.tq_split_attn_logits_workspace_bytes(hi, lo, L, N_Q, N_KV), dev)

        def fill():
            tq.tq_split_quantize_kv(hi, lo, Kx, hp, hn, lp, ln)

        def prepare():
            tq.tq_split_attn_prepare(hi, lo, q_all, L, N_Q, N_Q * D, N_KV, ws)

        def stream_only():
            tq.tq_split_attn_logits_prepared(hi, lo, ws, L, N_Q, hp, hn, lp, ln, N_KV, L * N_TOK,
                                             seq_start, seq_len, N_TOK, scale, logits, L * N_TOK)

        def one_call():
            tq.tq_split_attn_logits(hi, lo, q_all, L, N_Q, N_Q * D, hp, hn, lp, ln, N_KV,
                                    L * N_TOK, seq_start, seq_len, N_TOK, scale, logits,
                                    L * N_TOK, ws)

        fill()
        for _ in range(args.warmup):
            one_call()
        torch.cuda.synchronize()
        f_ms, _ = events(fill, 3)
        # the key stream alone, launched behind the query preparation as in a
        # decode step
        s_ms, s_med = events(stream_only, reps, before=prepare)
        # whole calls (preparation + stream) back to back
        t0 = time.perf_counter()
        for _ in range(args.steps):
            one_call()
        torch.cuda.synchronize()
        c_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        ows = tq.workspace(tq.tq_split_attn_output_workspace_bytes(hi, lo, L, N_Q, N_KV, N_TOK),
                           dev)

        def vout():
            tq.tq_split_attn_output(hi, lo, pw, L * N_TOK, L, N_Q, hp, hn, lp, ln, N_KV,
                                    L * N_TOK, seq_start, seq_len, N_TOK, out, N_Q * D, ows)

        vout()
        o_ms, o_med = events(vout, reps)
        rec = (DH * bh // 8 + 4) + (DH * bl // 8 + 4)
        alg = n_rec * rec + N_Q * L * N_TOK * 4
        bits = (DH * bh + DH * bl) / D
        res[f"{bits:g}"] = {
            "b_hi": bh, "b_lo": bl, "record_pair_bytes": rec,
            "logits_per_s": N_Q * L * N_TOK / (c_ms * 1e-3), "call_ms_mean": c_ms,
            "roofline": {"bound": "hbm", "kernel": f"attn_logits_res_kernel<{bh},false,4,{bl},true>",
                         "achieved": alg / (s_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": alg / (s_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": None, "alg_bytes_per_launch": alg,
                         "kernel_ms_mean": s_ms, "kernel_ms_median": s_med},
            "quantize_vec_per_s": n_rec / (f_ms * 1e-3), "quantize_ms": f_ms,
            "attn_output": {"ms_mean": o_ms, "ms_median": o_med,
                            "GB_per_s": alg / (o_ms * 1e-3) / 1e9,
                            "hbm_frac": alg / (o_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        hi.close()
        lo.close()
        del hp, lp, hn, ln, ws, ows
    return _line(args, "packed-key attention logits/sec at fractional bit widths (channel split)",
                 res["2.5"]["logits_per_s"], "logits/s",
                 {"workload": f"llama-3.1-8b decode layer x {L} layer caches (32 q / 8 kv heads, "
                              f"32768 tokens, d=128): channels 0-63 at b_hi, 64-127 at b_lo; "
                              f"value = 2.5-bit logits incl. query prep"},
                 {"dtype": "int8-mfma/fp32", "widths": res})


def run_long(args):
    """8 KV heads x 131072 tokens, b in {2, 3, 4}: quantize K+V, 32 x 131072 logits."""
    import torch
    import kv_cache_vector_pi_amd as tq
    import workloads
    dev, d, n_kv, n_q, n_tok = "cuda", 128, 8, 32, 131072
    stream = torch.cuda.current_stream()
    wl = workloads.long_context(dev)
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)     # 1 GiB

    def flush():
        flush_buf.fill_(0.0)

    per_b = {}
    reps = max(5, min(args.steps, 20))
    for b in _bits(args, [2, 3, 4], [1, 2, 3]):
        ctx = _common(args, d, b)
        rec = tq.tq_record_words(d, b)
        kp = torch.zeros((n_kv * n_tok, rec), dtype=torch.int32, device=dev)
        kn = torch.zeros((n_kv * n_tok, 2), dtype=torch.int16, device=dev)
        vp, vn = torch.zeros_like(kp), torch.zeros_like(kn)

        def quant():
            tq.tq_quantize_kv(ctx, wl["K"], kp, kn)
            tq.tq_quantize_kv(ctx, wl["V"], vp, vn)

        for _ in range(args.warmup):
            quant()
        q_ms, _ = _timed(quant, reps, stream, flush)
        logits = torch.empty((n_q, n_tok), dtype=torch.float32, device=dev)
        ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, 1, n_q, n_kv), dev)
        ss = torch.zeros(1, dtype=torch.int64, device=dev)
        sl = torch.full((1,), n_tok, dtype=torch.int32, device=dev)

        def logit():
            tq.tq_attn_logits(ctx, wl["q"], 1, n_q, n_q * d, kp, kn, n_kv, n_tok, ss, sl, n_tok,
                              1.0 / math.sqrt(d), logits, n_tok, ws)

        for _ in range(args.warmup):
            logit()
        l_ms, l_med = _timed(logit, reps, stream, flush)
        rb = b * d // 8 + 4
        n_vec = 2 * n_kv * n_tok
        per_b[str(b)] = {
            "quantize_vec_per_s": n_vec / (q_ms * 1e-3),
            "quantize_GB_per_s": n_vec * (2 * d + rb) / (q_ms * 1e-3) / 1e9,
            "logit_keys_per_s": n_kv * n_tok / (l_ms * 1e-3),
            "logits_per_s": n_q * n_tok / (l_ms * 1e-3),
            "logit_GB_per_s": n_kv * n_tok * (rb + 4 * (n_q // n_kv)) / (l_ms * 1e-3) / 1e9,
            "logit_ms_mean": l_ms, "logit_ms_median": l_med, "quantize_ms_mean": q_ms}
        ctx.close()
        del kp, kn, vp, vn
    top = per_b[max(per_b, key=int)]
    return _line(args, "packed-key attention logits/sec (long context, MALL-cold)",
                 top["logits_per_s"], "logits/s",
                 {"workload": "long context: 8 kv heads x 131072 tokens x 128, 32 q heads, "
                              "bf16 N(0,1) K/V; logits include query prep; a 1 GiB buffer is "
                              "written before each timed rep"},
                 {"dtype": "int8-mfma/fp32", "per_bits": per_b,
                  "peak_GB_per_s": HBM_PEAK_GBS})


def run_batched(args):
    """16 ragged sequences, b = 3: quantize a 512-token chunk per sequence,
    then logits for one 32-head query per sequence."""
    import torch
    import kv_cache_vector_pi_amd as tq
    import workloads
    dev, d, b = "cuda", 128, 3
    stream = torch.cuda.current_stream()
    wl = workloads.batched(dev)
    lens, chunk, n_kv, n_q = wl["lens"], wl["chunk"], wl["n_kv"], wl["n_q"]
    batch = len(lens)
    offs = [0]
    for n in lens[:-1]:
        offs.append(offs[-1] + n)
    total = sum(lens)
    ctx = _common(args, d, b)
    rec = tq.tq_record_words(d, b)
    kp = torch.zeros((n_kv * total, rec), dtype=torch.int32, device=dev)
    kn = torch.zeros((n_kv * total, 2), dtype=torch.int16, device=dev)
    vp, vn = torch.zeros_like(kp), torch.zeros_like(kn)
    K, V = wl["K"], wl["V"]
    for i in range(batch):                       # prefixes, untimed
        a, n = offs[i], lens[i] - chunk
        tq.tq_quantize_kv(ctx, K[:, a:a + n], kp, kn, dst_stride_head=total, dst_token0=a)
        tq.tq_quantize_kv(ctx, V[:, a:a + n], vp, vn, dst_stride_head=total, dst_token0=a)

    def quant_per_seq():
        for i in range(batch):
            a = offs[i] + lens[i] - chunk
            tq.tq_quantize_kv(ctx, K[:, a:a + chunk], kp, kn, dst_stride_head=total,
                              dst_token0=a)
            tq.tq_quantize_kv(ctx, V[:, a:a + chunk], vp, vn, dst_stride_head=total,
                              dst_token0=a)

    # the chunks of all sequences as one input, as a model's projection emits
    # the new tokens of a batch together, with each token's destination
    idx = torch.cat([torch.arange(o + n - chunk, o + n) for o, n in zip(offs, lens)]).to(dev)
    Kn, Vn = K[:, idx].contiguous(), V[:, idx].contiguous()

    def quant():
        tq.tq_quantize_kv_slots(ctx, Kn, idx, kp, kn, total)
        tq.tq_quantize_kv_slots(ctx, Vn, idx, vp, vn, total)

    ss = torch.tensor(offs, dtype=torch.int64, device=dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    logits = torch.empty((n_q, total), dtype=torch.float32, device=dev)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, batch, n_q, n_kv), dev)

    def logit():
        tq.tq_attn_logits(ctx, wl["q"], batch, n_q, n_q * d, kp, kn, n_kv, total, ss, sl,
                          max(lens), 1.0 / math.sqrt(d), logits, total, ws)

    reps = max(5, min(args.steps, 50))
    for _ in range(args.warmup):
        quant_per_seq()
        quant()
        logit()
    qs_ms, _ = _timed(quant_per_seq, reps, stream)
    q_ms, _ = _timed(quant, reps, stream)
    l_ms1, l_med1 = _timed(logit, reps, stream)
    # calls back to back, as in a serving loop (the launch of one call
    # overlaps the previous one): the throughput figure
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        logit()
    ev1.record(stream)
    ev1.synchronize()
    l_ms = ev0.elapsed_time(ev1) / reps
    rb = b * d // 8 + 4
    alg = n_kv * total * (rb + 4 * (n_q // n_kv))
    ctx.close()
    return _line(args, "packed-key attention logits/sec (batched ragged decode)",
                 n_q * total / (l_ms * 1e-3), "logits/s",
                 {"workload": f"batched decode: {batch} sequences, lengths {min(lens)}..{max(lens)} "
                              f"(total {total}), 8 kv / 32 q heads, d=128, b=3; quantize a "
                              f"512-token chunk per sequence (K and V, slot-mapped), logits "
                              f"include query prep"},
                 {"dtype": "int8-mfma/fp32", "logit_ms_back_to_back": l_ms,
                  "logit_ms_single_call_mean": l_ms1, "logit_ms_single_call_median": l_med1,
                  "logit_keys_per_s": n_kv * total / (l_ms * 1e-3),
                  "logit_GB_per_s": alg / (l_ms * 1e-3) / 1e9,
                  "logit_hbm_frac": alg / (l_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "chunk_quantize_ms": q_ms,
                  "chunk_quantize_vec_per_s": 2 * n_kv * chunk * batch / (q_ms * 1e-3),
                  "chunk_quantize_form": "tq_quantize_kv_slots, one call each for K and V",
                  "chunk_quantize_per_sequence_calls_ms": qs_ms})


def run_attn_out(args):
    """tq_attn_output over the packed values of 32 Llama-shaped layer caches
    (8 KV heads x 32768 tokens, b = 4), one launch pair for all layers."""
    import torch
    import kv_cache_vector_pi_amd as tq
    import workloads
    dev, d, n_kv, n_q, n_tok, L = "cuda", 128, 8, 32, 32768, args.layers
    b = _bits(args, [4], [3])[0]
    stream = torch.cuda.current_stream()
    ctx = _common(args, d, b)
    rw = tq.tq_record_words(d, b)
    vp = torch.zeros((n_kv * L * n_tok, rw), dtype=torch.int32, device=dev)
    vn = torch.zeros((n_kv * L * n_tok, 2), dtype=torch.int16, device=dev)
    Vx = torch.empty((n_kv, L * n_tok, d), dtype=torch.bfloat16, device=dev)
    for l in range(L):
        Vx[:, l * n_tok:(l + 1) * n_tok] = workloads.llama(dev, seed=l, n_tok=n_tok)["V"]
    tq.tq_quantize_kv(ctx, Vx, vp, vn)
    del Vx
    g = workloads.gen(0, workloads.STREAM_Q, dev)
    p = torch.softmax(torch.randn((n_q, L * n_tok), generator=g, device=dev).view(n_q, L, n_tok),
                      dim=2).view(n_q, L * n_tok).contiguous()
    seq_start = torch.arange(L, dtype=torch.int64, device=dev) * n_tok
    seq_len = torch.full((L,), n_tok, dtype=torch.int32, device=dev)
    out = torch.empty((L, n_q, d), device=dev)
    ws = tq.workspace(tq.tq_attn_output_workspace_bytes(ctx, L, n_q, n_kv, n_tok), dev)

    def run():
        tq.tq_attn_output(ctx, p, L * n_tok, L, n_q, vp, vn, n_kv, L * n_tok, seq_start, seq_len,
                          n_tok, out, n_q * d, ws)

    for _ in range(max(1, args.warmup)):
        run()
    ms, med = _timed(run, max(5, min(args.steps, 50)), stream)
    rec = n_kv * L * n_tok
    alg = rec * (b * d // 8 + 4) + n_q * L * n_tok * 4           # values + weights read
    ctx.close()
    return _line(args, "attention output from packed values: values/sec", rec / (ms * 1e-3),
                 "values/s",
                 {"workload": "llama-3.1-8b decode layer values: 8 kv / 32 q heads, d=128, "
                              f"32768 tokens, b={b}; 32 layer caches per launch"},
                 {"dtype": "f32", "ms_mean": ms, "ms_median": med,
                  "GB_per_s": alg / (ms * 1e-3) / 1e9,
                  "hbm_frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "alg_bytes_per_call": alg})


def run_decode_fused(args):
    """tq_attn_decode over 32 Llama-shaped layer caches (8 KV heads x 32768
    tokens, b = 4, K and V packed), one call for all layers."""
    import torch
    import kv_cache_vector_pi_amd as tq
    import workloads
    dev, d, n_kv, n_q, n_tok, L = "cuda", 128, 8, 32, 32768, args.layers
    b = _bits(args, [4], [3])[0]
    stream = torch.cuda.current_stream()
    ctx = _common(args, d, b)
    rw = tq.tq_record_words(d, b)
    kp = torch.zeros((n_kv * L * n_tok, rw), dtype=torch.int32, device=dev)
    kn = torch.zeros((n_kv * L * n_tok, 2), dtype=torch.int16, device=dev)
    vp, vn = torch.zeros_like(kp), torch.zeros_like(kn)
    for l in range(L):
        wl = workloads.llama(dev, seed=l, n_tok=n_tok)
        tq.tq_quantize_kv(ctx, wl["K"], kp, kn, dst_stride_head=L * n_tok, dst_token0=l * n_tok)
        tq.tq_quantize_kv(ctx, wl["V"], vp, vn, dst_stride_head=L * n_tok, dst_token0=l * n_tok)
        del wl
    q_all = torch.stack([workloads.normal((n_q, d), l, workloads.STREAM_Q, dev) for l in range(L)])
    seq_start = torch.arange(L, dtype=torch.int64, device=dev) * n_tok
    seq_len = torch.full((L,), n_tok, dtype=torch.int32, device=dev)
    out = torch.empty((L, n_q, d), device=dev)
    ws = tq.workspace(tq.tq_attn_decode_workspace_bytes(ctx, L, n_q, n_kv, n_tok), dev)

    def run():
        tq.tq_attn_decode(ctx, q_all, L, n_q, n_q * d, kp, kn, vp, vn, n_kv, L * n_tok, seq_start,
                          seq_len, n_tok, 1.0 / math.sqrt(d), out, n_q * d, ws)

    for _ in range(max(1, args.warmup)):
        run()
    ms, med = _timed(run, max(5, min(args.steps, 50)), stream)
    rec = n_kv * L * n_tok
    alg = 2 * rec * (b * d // 8 + 4)                 # keys and values read once
    ctx.close()
    return _line(args, "fused decode attention from packed K/V: tokens/sec (all heads)",
                 L * n_tok / (ms * 1e-3), "tokens/s",
                 {"workload": "llama-3.1-8b decode layer: 8 kv / 32 q heads, d=128, 32768 "
                              f"cached tokens, b={b} K and V; 32 layer caches per call"},
                 {"dtype": "int8-mfma/fp32", "ms_mean": ms, "ms_median": med,
                  "GB_per_s": alg / (ms * 1e-3) / 1e9,
                  "hbm_frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "alg_bytes_per_call": alg})


def run_search(args):
    """1e6 unit vectors at d (1536 or 200), b in {2, 4}: quantize the
    database, then top-10 of 1000 queries over all of it."""
    import torch
    import kv_cache_vector_pi_amd as tq
    import workloads
    dev, d, k = "cuda", args.search_d, 10
    stream = torch.cuda.current_stream()
    wl = workloads.search(dev, d)
    db, qs = wl["db"], wl["queries"]
    n_db, n_q = db.shape[0], qs.shape[0]
    # exact float top-10 for the recall diagnostic
    exact = torch.empty((n_q, k), dtype=torch.int64, device=dev)
    best = torch.full((n_q, k), -float("inf"), device=dev)
    for c0 in range(0, n_db, 131072):
        sc = qs @ db[c0:c0 + 131072].T
        cand_s = torch.cat([best, sc], dim=1)
        cand_i = torch.cat([exact, torch.arange(c0, c0 + sc.shape[1], device=dev)
                            .expand(n_q, -1)], dim=1)
        best, pos = cand_s.topk(k, dim=1)
        exact = torch.gather(cand_i, 1, pos)
    per_b = {}
    reps = max(3, min(args.steps, 10))
    for b in _bits(args, [2, 4], [2, 3]):
        ctx = _common(args, d, b)
        planes, norms = tq.alloc_records(n_db, d, b, dev)
        # blocked products with a workspace at large d (none needed at d = 200)
        qws_bytes = tq.tq_quantize_workspace_bytes(ctx, n_db)
        qws = tq.workspace(qws_bytes, dev) if qws_bytes else None

        def quant():
            tq.tq_quantize_kv_ws(ctx, db, planes, norms, qws)

        for _ in range(max(1, args.warmup)):
            quant()
        q_ms, _ = _timed(quant, reps, stream)
        ws = tq.workspace(tq.tq_search_workspace_bytes(ctx, n_q, n_db, k), dev)
        oi = torch.empty((n_q, k), dtype=torch.int64, device=dev)
        osc = torch.empty((n_q, k), dtype=torch.float32, device=dev)

        def search():
            tq.tq_search_topk(ctx, qs, n_q, planes, norms, n_db, k, oi, osc, ws)

        for _ in range(max(1, args.warmup)):
            search()
        s_ms, s_med = _timed(search, reps, stream)
        hit = sum(len(set(a) & set(e)) for a, e in zip(oi.cpu().tolist(), exact.cpu().tolist()))
        pairs = n_q * n_db
        rb = b * d // 8 + 4
        per_b[str(b)] = {
            "quantize_vec_per_s": n_db / (q_ms * 1e-3),
            "quantize_GB_per_s": n_db * (4 * d + rb) / (q_ms * 1e-3) / 1e9,
            "quantize_ms": q_ms,
            "search_ms_mean": s_ms, "search_ms_median": s_med,
            "scores_per_s": pairs / (s_ms * 1e-3),
            "queries_per_s": n_q / (s_ms * 1e-3),
            "alg_TFLOP_per_s": 4 * d * pairs / (s_ms * 1e-3) / 1e12,
            "alg_frac_of_fp16_mfma": 4 * d * pairs / (s_ms * 1e-3) / 2.5e15,
            "recall_at_10_vs_exact_fp32": hit / (n_q * k)}
        ctx.close()
        del planes, norms, ws
    top = per_b[max(per_b, key=int)]
    return _line(args, "vector search: scores/sec from packed codes (top-10)",
                 top["scores_per_s"], "scores/s",
                 {"workload": f"vector search: {n_db} unit vectors (normalised N(0,I)) at d={d}, "
                              f"{n_q} queries, top-{k}; fp32 input"},
                 {"dtype": "fp16-mfma/fp32", "per_bits": per_b})


if __name__ == "__main__":
    main()
