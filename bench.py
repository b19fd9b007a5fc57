"""Benchmark of the absorbed MLA decode step on one MI355X.

One step = the whole hot path on one batch of synthetic input already resident
in HBM: absorb W^UK, latent attention (split over positions), merge of the
splits, W^UV — by default the one call mla_decode_step, which fuses the split
merge into W^UV; with --three-calls the separate calls mla_absorb_q ->
mla_decode_latent_attn -> mla_out_up. For the fp8 sparse workload the weights
are dequantised once before timing, as the method memoises them. Default
workload: B=32, n_h=128, T=4096 cached positions, bf16, 1 query token per
sequence.

Timing: W untimed warm-up steps, then K timed steps bracketed by
synchronisation, HIP events on the stream the kernels run on, replayed from
HIP graphs of >= 60 steps (one per layer of a 61-layer decode graph). Each
step uses the next of R device replicas of the inputs (cache and weights each
>= 1.1 GB in total) so the 256 MB Infinity Cache cannot serve them. The roofline object reports the stand-alone attention call
(split + merge kernels; with whole 128-head groups on the packed queries the
step's attention kernel reads), timed per call from graphs of R and 3R
calls.

Prints ONE JSON line (metric/value/unit/..., roofline, cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

METRIC = "MLA absorbed decode: cached token·heads/s and % of HBM/MFMA roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--dequant", action="store_true",
                    help="time the one-time fp8 block dequantisation of the sparse "
                         "workload's wkv_b ([32768, 512] e4m3 + [256, 4] fp32 scales -> bf16)")
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5, 6, 7],
                    help="2: decode B=32 T=4096 (default); 3: decode B=4 T=32768; "
                         "4: sparse top-2048 decode with fp8 weights; 5: KV reconstruction "
                         "N=8192; 6: cache append of a 4 x 8192-token prefill; 7: naive-path "
                         "causal attention over reconstructed K/V, S=T=8192, 128 heads")
    ap.add_argument("--min-replica-bytes", type=float, default=1.1e9)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--three-calls", action="store_true",
                    help="run the decode step as three library calls (absorb, attention with "
                         "its split merge, W^UV) instead of the one-call mla_decode_step")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of HIP-graph replays of the step")
    ap.add_argument("--tp", type=int, default=1, metavar="G",
                    help="one GPU's tensor-parallel share of a decode workload: 128/G heads "
                         "(the whole cache is still read)")
    ap.add_argument("--splits", type=int, default=0, metavar="S",
                    help="decode workloads: split the attended positions of each sequence into "
                         "S parts (0: the library's automatic plan)")
    ap.add_argument("--yarn", action="store_true",
                    help="use the context-extended (YaRN) attention scale: "
                         "max_seq_len 163840 > 4096, mscale 1, rope_factor 40")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes three times "
                         "(the reference kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return ap.parse_args()


def algorithmic_work(B, n_h, rows, esz=2):
    """Bytes that must move and flops that must happen (intermediates q_lat,
    o_lat and split partials excluded). rows = attended positions/sequence."""
    cache = B * rows * 576 * esz
    w = n_h * 256 * 512 * esz
    q = B * n_h * (128 + 64) * esz
    out = B * n_h * 128 * esz
    q_lat = B * n_h * 512 * esz
    o_lat = B * n_h * 512 * esz
    q_pe = B * n_h * 64 * esz
    step_bytes = cache + w + q + out
    attn_bytes = cache + q_lat + q_pe + o_lat
    attn_flops = B * rows * n_h * (576 + 512) * 2
    step_flops = attn_flops + 2 * B * n_h * 128 * 512 * 2
    return dict(step_bytes=step_bytes, step_flops=step_flops, attn_bytes=attn_bytes,
                attn_flops=attn_flops, cache_bytes=cache, w_bytes=w)


def roofline_time_s(nbytes, flops):
    return max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFS * 1e12))


def traffic_record(kernel_key):
    """HBM bytes per launch from committed rocprofv3 counter runs
    (profiles/traffic.json), if they were taken on the current kernel
    sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, "head_latent_attention_mla_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    return rec["bytes_per_launch"] if h.hexdigest()[:16] == rec["sources_sha256_16"] else None


def cpu_baseline(cfg, inp):
    """The fp64 oracle (as written, untuned) on the same workload, host cores."""
    import numpy as np  # noqa: F401
    import oracle
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    cache = inp["cache"]
    B = cache.shape[0]
    nb = B  # whole batch: 10-30 s of CPU work on a 16-core host share
    if cfg == 4:
        w = inp["wkv_b_ref"]
        topk = inp["topk_idx"][:nb]
    else:
        w = inp["wkv_b"]
        topk = None
    t0 = time.perf_counter()
    oracle.decode_absorbed(inp["q_nope"][:nb], inp["q_pe"][:nb], cache[:nb, :, :512],
                           cache[:nb, :, 512:], w, topk_idx=topk)
    dt = time.perf_counter() - t0
    n_h = inp["q_nope"].shape[1]
    rows = topk.shape[1] if topk is not None else cache.shape[1]
    return {"value": nb * rows * n_h / dt, "unit": "cached token·heads/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"one full decode step of {nb} sequences x {rows} positions x {n_h} heads, "
                      f"fp64 C oracle, OpenMP over (sequence, head)"}


INPUT_NOTE = ("latent rows of unit RMS (512 standard normals scaled to RMS 1: how an "
              "RMS-normalised standard normal row with unit gain is distributed), rotary "
              "keys and queries N(0,1), wkv_b N(0,1/512)")


def batch_stats(torch, replay, n_batches, steps_per_batch):
    """Per-step time of each of n_batches back-to-back replays (events
    between replays on the stream the work runs on): median, p10, p90 in
    microseconds."""
    import numpy as np
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_batches + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(n_batches):
        replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(n_batches)]) * 1e3
    per /= steps_per_batch
    return {"median_us": float(np.median(per)), "p10_us": float(np.percentile(per, 10)),
            "p90_us": float(np.percentile(per, 90)), "batches": n_batches,
            "steps_per_batch": steps_per_batch}


def time_single_call(args, torch, call, R):
    """Workloads of one library call per step. Returns (per-call ms, step ms).

    Per-call duration: graphs of R and 3R back-to-back calls (one per input
    replica), the difference divided by 2R, which cancels the fixed cost of
    launching a graph; with --no-graph, events around eager launches.
    Timed region: exactly K calls bracketed by synchronisation, replayed from
    graphs of R calls plus one graph of the K mod R rest (or launched eagerly
    with --no-graph)."""
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()

    def events():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    if args.no_graph:
        e0, e1 = events()
        e0.record()
        for i in range(args.steps):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        time_single_call.stats = None
        return ms, ms

    def graph_of(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                call(i)
        g.replay()
        torch.cuda.synchronize()
        return g

    def replay_ms(g, rounds):
        e0, e1 = events()
        e0.record()
        for _ in range(rounds):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    g1, g3 = graph_of(R), graph_of(3 * R)
    rounds = max(2, args.steps // (2 * R))
    call_ms = (replay_ms(g3, rounds) - replay_ms(g1, rounds)) / (rounds * 2 * R)
    full, rest = divmod(args.steps, R)
    g_rest = graph_of(rest) if rest else None
    torch.cuda.synchronize()
    e0, e1 = events()
    e0.record()
    for _ in range(full):
        g1.replay()
    if g_rest is not None:
        g_rest.replay()
    e1.record()
    torch.cuda.synchronize()
    time_single_call.stats = batch_stats(torch, g1.replay, max(20, full), R)
    return call_ms, e0.elapsed_time(e1) / args.steps


def reconstruct_main(args, torch, mla, synth):
    """Config 5: the naive path's KV reconstruction, one call per step."""
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[5]
    N, n_h = cfg["N"], cfg["n_h"]
    inp = synth.config_inputs(5)
    base = {k: v.to(dev) for k, v in inp.items()}
    per_rep = sum(v.numel() * v.element_size() for v in base.values())
    w_bytes = base["wkv_b"].numel() * base["wkv_b"].element_size()
    # (the weights alone also above the bound: see the decode replicas)
    R = max(2, int(-(-args.min_replica_bytes // per_rep)),
            int(-(-args.min_replica_bytes // w_bytes)))
    reps = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
    K = torch.empty((N, n_h, 192), dtype=torch.bfloat16, device=dev)
    V = torch.empty((N, n_h, 128), dtype=torch.bfloat16, device=dev)

    def step(i):
        x = reps[i % R]
        mla.mla_kv_reconstruct(x["c"], x["k_rope"], x["wkv_b"], K, V)

    call_ms, ms = time_single_call(args, torch, step, R)
    nbytes = (N * 512 + N * 64 + n_h * 256 * 512 + N * n_h * (192 + 128)) * 2
    flops = 2 * N * 512 * n_h * 256
    tflops = flops / (call_ms * 1e-3) / 1e12
    line = {
        "metric": "MLA KV reconstruction: token·heads/s and % of MFMA roofline",
        "value": N * n_h / (ms * 1e-3), "unit": "token·heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; no datasets or trained weights)",
        "config": {"workload": cfg["name"], "N": N, "n_h": n_h, "input_replicas": R},
        "roofline": {"bound": "mfma", "kernel": "mla_kv_reconstruct", "achieved": tflops,
                     "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFS,
                     "traffic": traffic_record("reconstruct_config5"),
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": call_ms * 1e3,
                     "roofline_us": roofline_time_s(nbytes, flops) * 1e6},
        "published_baseline": "none: the source pages print no throughput figures",
        "step_stats": time_single_call.stats,
    }
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        n = 64  # rows of the sample: about 10-30 s of fp64 work on the host
        t = time.perf_counter()
        oracle.kv_reconstruct(inp["c"][:n], inp["k_rope"][:n], inp["wkv_b"], n_h)
        dt = time.perf_counter() - t
        line["cpu_baseline"] = {"value": n * n_h / dt, "unit": "token·heads/s", "cores": cores,
                                "kind": "oracle", "seconds": round(dt, 3),
                                "sample": f"{n} of the {N} tokens, all {n_h} heads, fp64 C oracle"}
    print(json.dumps(line))


def append_main(args, torch, mla, synth):
    """Cache append (RMSNorm of the latent, rotation of the rotary key, write
    into the packed cache) of a prefill: B=4 sequences x 8192 new tokens into
    a [4, 32768, 576] bf16 cache. One call per step; HIP graphs of R and 3R
    calls, the difference giving the per-call duration."""
    dev = torch.device("cuda:0")
    B, per, T = 4, 8192, 32768
    N = B * per
    inp = synth.append_inputs(N, B, T, torch.bfloat16, seed=1006, prefill=True)
    base = {k: v.to(dev) for k, v in inp.items()}
    cache = torch.zeros((B, T, 576), dtype=torch.bfloat16, device=dev)
    per_rep = sum(v.numel() * v.element_size() for v in base.values())
    R = max(2, int(-(-args.min_replica_bytes // per_rep)))
    reps = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]

    def call(i):
        x = reps[i % R]
        mla.mla_cache_append(x["kv_a"], x["gamma"], x["freqs"], x["pos"], cache[..., :512],
                             cache[..., 512:], seq_idx=x["seq_idx"])

    call_ms, ms = time_single_call(args, torch, call, R)
    # algorithmic bytes per row: 576 bf16 in, 576 bf16 out, the 256-byte
    # (cos, sin) table row, two int32 indices; plus the 2 KB gain once
    nbytes = N * (576 * 2 * 2 + 256 + 8) + 512 * 4
    gbs = nbytes / (call_ms * 1e-3) / 1e9
    line = {
        "metric": "MLA cache append: rows/s and % of HBM roofline",
        "value": N / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; no datasets or trained weights)",
        "config": {"workload": "cache append bf16, prefill of B=4 x 8192 tokens into a "
                               "[4, 32768, 576] packed cache", "N": N, "input_replicas": R},
        "roofline": {"bound": "hbm", "kernel": "mla_cache_append", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": traffic_record("append_config6"),
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": call_ms * 1e3},
        "published_baseline": "none: the source pages print no throughput figures",
        "step_stats": time_single_call.stats,
    }
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        kv = inp["kv_a"]
        t = time.perf_counter()
        oracle.cache_append(kv[:, :512].contiguous(), kv[:, 512:].contiguous(), inp["gamma"],
                            inp["freqs"], inp["pos"])
        dt = time.perf_counter() - t
        line["cpu_baseline"] = {"value": N / dt, "unit": "rows/s", "cores": 1,
                                "kind": "oracle", "seconds": round(dt, 3),
                                "sample": f"all {N} rows, fp64 C oracle, one thread"}
    print(json.dumps(line))


def attention_main(args, torch, mla, synth):
    """Naive path, second half: causal attention of an 8192-token prefill
    over its reconstructed keys and values (128 heads, bf16). One call per
    step; HIP graphs of R and 3R calls give the per-call duration."""
    dev = torch.device("cuda:0")
    B, S, T, n_h = 1, 8192, 8192, 128
    inp = synth.attention_inputs(B, S, T, n_h, torch.bfloat16, seed=1007)
    base = {k: v.to(dev) for k, v in inp.items()}
    out = torch.empty((B, S, n_h, 128), dtype=torch.bfloat16, device=dev)
    # the working set (1.1 GB) is far beyond the caches: two replicas suffice
    R = 2
    reps = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]

    def call(i):
        x = reps[i % R]
        mla.mla_attention_naive(x["q"], x["k"], x["v"], causal=True, out=out)

    call_ms, ms = time_single_call(args, torch, call, R)
    # algorithmic work: every visible (query, key) pair once, 192-deep score
    # and 128-deep value product per head; bytes: q, k, v in, out out
    pairs = S * (S + 1) // 2 if S == T else S * T
    flops = pairs * n_h * (192 + 128) * 2
    nbytes = (B * S * n_h * (192 + 128) + B * T * n_h * (192 + 128)) * 2
    tfs = flops / (call_ms * 1e-3) / 1e12
    line = {
        "metric": "MLA naive-path attention: query·heads/s and % of MFMA roofline",
        "value": B * S * n_h / (ms * 1e-3), "unit": "query·heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; no datasets or trained weights)",
        "config": {"workload": "causal attention bf16 over reconstructed K/V, B=1 S=T=8192 "
                               "n_h=128 (192-feature keys, 128-feature values)",
                   "B": B, "S": S, "T": T, "n_h": n_h, "input_replicas": R},
        "roofline": {"bound": "mfma", "kernel": "mla_attention_naive", "achieved": tfs,
                     "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": tfs / MFMA_BF16_PEAK_TFS,
                     "traffic": traffic_record("attention_config7"),
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": call_ms * 1e3,
                     "roofline_us": roofline_time_s(nbytes, flops) * 1e6},
        "published_baseline": "none: the source pages print no throughput figures",
        "step_stats": time_single_call.stats,
    }
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(cores))
        # the last 16 queries (the most keys each), all heads
        nq = 16
        t = time.perf_counter()
        oracle.attention_naive(inp["q"][:, S - nq:], inp["k"], inp["v"], causal=True)
        dt = time.perf_counter() - t
        line["cpu_baseline"] = {"value": nq * n_h / dt, "unit": "query·heads/s",
                                "cores": cores, "kind": "oracle", "seconds": round(dt, 3),
                                "sample": f"the last {nq} of the {S} queries (8177..8192 keys "
                                          f"each), all {n_h} heads, fp64 C oracle, OpenMP"}
    print(json.dumps(line))


def dequant_main(args, torch, mla, synth):
    """The one-time fp8 block dequantisation of the sparse workload's wkv_b:
    [32768, 512] e4m3 codes with one fp32 scale per 128x128 block -> bf16.
    One call per step; HIP graphs of R and 3R calls (one per input replica)
    give the per-call duration."""
    dev = torch.device("cuda:0")
    inp = synth.config_inputs(4)
    codes = inp["wkv_b_fp8"].to(dev)
    scales = inp["wkv_b_scale"].to(dev)
    rows, cols = codes.shape
    nbytes = rows * cols * (1 + 2) + scales.numel() * 4  # codes in, bf16 out, scales
    R = max(2, int(-(-args.min_replica_bytes // nbytes)))
    reps = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(R - 1)]
    outs = [torch.empty((rows, cols), dtype=torch.bfloat16, device=dev) for _ in range(R)]

    def call(i):
        c, sc = reps[i % R]
        mla.mla_dequant_fp8_block(c, sc, out=outs[i % R])

    call_ms, ms = time_single_call(args, torch, call, R)
    gbs = nbytes / (call_ms * 1e-3) / 1e9
    line = {
        "metric": "MLA fp8 block dequantisation of wkv_b: weights/s and % of HBM roofline",
        "value": rows * cols / (ms * 1e-3), "unit": "weights/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3->bf16",
        "data": "synthetic (seeded; no datasets or trained weights)",
        "config": {"workload": "fp8 e4m3 block dequantisation of wkv_b [32768, 512] "
                               "(one fp32 scale per 128x128 block, scales U[0.5,2]*2^-4) to bf16",
                   "rows": rows, "cols": cols, "input_replicas": R},
        "roofline": {"bound": "hbm", "kernel": "mla_dequant_fp8_block", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": traffic_record("dequant_config4"),
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": call_ms * 1e3,
                     "roofline_us": nbytes / (HBM_PEAK_GBS * 1e9) * 1e6},
        "published_baseline": "none: the source pages print no throughput figures",
        "step_stats": time_single_call.stats,
    }
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(cores))
        t = time.perf_counter()
        oracle.dequant_fp8_block(inp["wkv_b_fp8"].numpy(), inp["wkv_b_scale"].numpy())
        dt = time.perf_counter() - t
        line["cpu_baseline"] = {"value": rows * cols / dt, "unit": "weights/s", "cores": cores,
                                "kind": "oracle", "seconds": round(dt, 3),
                                "sample": f"the whole [{rows}, {cols}] weight, fp64 C oracle, "
                                          f"OpenMP over rows"}
    print(json.dumps(line))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU runs are not "
                          "supported (--gpus must be 1)", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from head_latent_attention_mla_amd import binding as mla
    from head_latent_attention_mla_amd import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.copy_probe:
        src = torch.ones(args.copy_probe, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe}))
        return
    if args.dequant:
        return dequant_main(args, torch, mla, synth)
    if args.config == 5:
        return reconstruct_main(args, torch, mla, synth)
    if args.config == 6:
        return append_main(args, torch, mla, synth)
    if args.config == 7:
        return attention_main(args, torch, mla, synth)
    dev = torch.device("cuda:0")
    cfg = dict(synth.CONFIGS[args.config])
    if args.tp > 1:
        if 128 % args.tp:
            print(json.dumps({"error": "--tp must divide 128"}))
            sys.exit(2)
        cfg["n_h"] = 128 // args.tp
        cfg["name"] += f", tensor-parallel share n_h=128/{args.tp}"
    B, n_h, T = cfg["B"], cfg["n_h"], cfg["T"]
    inp = synth.config_inputs(args.config, n_h=n_h)
    scale = (mla.mla_softmax_scale(192, 163840, 4096, 1.0, 40.0) if args.yarn
             else mla.mla_softmax_scale(192))
    sparse = "topk_idx" in inp
    rows = inp["topk_idx"].shape[1] if sparse else T

    # device replicas (inputs resident in HBM before timing)
    if args.config == 4:
        w0 = mla.mla_dequant_fp8_block(inp["wkv_b_fp8"].to(dev), inp["wkv_b_scale"].to(dev))
        torch.cuda.synchronize()
        inp["wkv_b_ref"] = w0.cpu()
    else:
        w0 = inp["wkv_b"].to(dev)
    base = dict(cache=inp["cache"].to(dev), q_nope=inp["q_nope"].to(dev),
                q_pe=inp["q_pe"].to(dev), w=w0,
                topk=inp["topk_idx"].to(dev) if sparse else None)
    per_rep = (base["cache"].numel() * 2 + w0.numel() * 2 if not sparse
               else B * rows * 576 * 2 + w0.numel() * 2)
    # enough replicas that the weights alone also exceed the bound: the cache
    # rows are read with the non-temporal hint, so a few replicas' weights
    # could otherwise stay in the 256 MB Infinity Cache from one round to the
    # next (a model's layers each have their own wkv_b)
    R = max(2, int(-(-args.min_replica_bytes // per_rep)),
            int(-(-args.min_replica_bytes // (w0.numel() * 2))))
    reps = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()}
                     for _ in range(R - 1)]
    q_lat = torch.empty((B, n_h, 512), dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty((B, n_h, 512), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, n_h, 128), dtype=torch.bfloat16, device=dev)
    K = rows if sparse else 0
    ws_bytes = mla.mla_decode_workspace_bytes(B, n_h, T, K, args.splits)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    splits = args.splits or mla.mla_decode_num_splits(B, n_h, T, K)

    step_ws_bytes = mla.mla_decode_step_workspace_bytes(B, 1, n_h, T, K, args.splits)
    step_ws = torch.empty(max(step_ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step(r, ev=None):
        x = reps[r % R]
        if ev is not None:
            ev[0].record()
        if args.three_calls:
            mla.mla_absorb_q(x["q_nope"], x["w"], q_lat)
            mla.mla_decode_latent_attn(q_lat, x["q_pe"], x["cache"][..., :512],
                                       x["cache"][..., 512:], topk_idx=x["topk"], scale=scale,
                                       num_splits=args.splits, out_lat=o_lat, workspace=ws)
            mla.mla_out_up(o_lat, x["w"], out)
        else:
            # one call: absorb, split attention, split merge fused into W^UV
            mla.mla_decode_step(x["q_nope"], x["q_pe"], x["w"], x["cache"][..., :512],
                                x["cache"][..., 512:], topk_idx=x["topk"], scale=scale,
                                num_splits=args.splits, out=out, workspace=step_ws)
        if ev is not None:
            ev[1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # eager pass: events around each step
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    eager_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps

    # per-call durations without host launch overhead: one HIP graph per call
    # kind holding that call once per replica, replayed; events on the stream
    # the graph (and so the kernels) run on
    # whole 128-head groups: the packed (operand-order) queries the one-call
    # step uses; the attention call is then the step's attention kernel plus
    # the stand-alone split merge
    packed = n_h % 128 == 0

    def call_absorb(r):
        x = reps[r]
        if packed:
            mla.mla_absorb_q_packed(x["q_nope"], x["w"], q_lat.view(B, -1))
        else:
            mla.mla_absorb_q(x["q_nope"], x["w"], q_lat)

    def call_decode(r):
        x = reps[r]
        if packed:
            mla.mla_decode_latent_attn_packed(q_lat.view(B, -1), x["q_pe"], x["cache"][..., :512],
                                              x["cache"][..., 512:], topk_idx=x["topk"],
                                              scale=scale, num_splits=args.splits,
                                              out_lat=o_lat, workspace=ws)
        else:
            mla.mla_decode_latent_attn(q_lat, x["q_pe"], x["cache"][..., :512],
                                       x["cache"][..., 512:], topk_idx=x["topk"], scale=scale,
                                       num_splits=args.splits, out_lat=o_lat, workspace=ws)

    def call_out_up(r):
        x = reps[r]
        mla.mla_out_up(o_lat, x["w"], out)

    def graph_of(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i % R)
        g.replay()
        torch.cuda.synchronize()
        return g

    def replay_ms(g, rounds):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(rounds):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def graph_call_ms(fn):
        # graphs of R and 3R calls: the difference cancels the fixed cost of
        # launching a graph, leaving back-to-back kernel execution per call
        g1, g3 = graph_of(fn, R), graph_of(fn, 3 * R)
        rounds = max(2, args.steps // (2 * R))
        return (replay_ms(g3, rounds) - replay_ms(g1, rounds)) / (rounds * 2 * R)

    if args.no_graph:
        # eager launches with events around each call (counter runs see
        # every dispatch)
        def eager_call_ms(fn):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(args.steps):
                fn(i % R)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps
        absorb_ms = eager_call_ms(call_absorb)
        decode_ms = eager_call_ms(call_decode)
        outup_ms = eager_call_ms(call_out_up)
    else:
        absorb_ms = graph_call_ms(call_absorb)
        decode_ms = graph_call_ms(call_decode)
        outup_ms = graph_call_ms(call_out_up)

    # timed region: exactly K whole steps, bracketed by synchronisation,
    # replayed from HIP graphs of G consecutive steps cycling over the R input
    # replicas, plus one graph for the remaining K mod G steps; G is whole
    # rounds over the replicas, at least 60 steps (a decode graph of a
    # 61-layer model holds one attention step per layer), so the fixed cost
    # of launching a graph is spread as it would be there
    G = R * max(1, -(-60 // R))
    full, rest = divmod(args.steps, G)
    if not args.no_graph:
        g_full = graph_of(step, G)
        g_rest = graph_of(step, rest) if rest else None
        for _ in range(max(1, args.warmup // G)):
            g_full.replay()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    if args.no_graph:
        for i in range(args.steps):
            step(i)
    else:
        for _ in range(full):
            g_full.replay()
        if g_rest is not None:
            g_rest.replay()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    # spread of the per-step time over >= 20 batches of R steps
    stats = None if args.no_graph else batch_stats(torch, g_full.replay, max(20, full), G)

    work = algorithmic_work(B, n_h, rows)
    value = B * rows * n_h / (ms_step * 1e-3)
    t_roof_step = roofline_time_s(work["step_bytes"], work["step_flops"])
    # dominant kernel: the latent attention call (split kernel + merge kernel)
    attn_gbs = work["attn_bytes"] / (decode_ms * 1e-3) / 1e9
    traffic = traffic_record(f"decode_config{args.config}" + (f"_tp{args.tp}" if args.tp > 1 else ""))
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "cached token·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no datasets or trained weights)",
        "config": {"workload": cfg["name"], "B": B, "n_h": n_h, "T": T, "tp_share": args.tp,
                   "attention_scale": scale,
                   "attended_positions": rows, "query_tokens": 1,
                   "fp8_weights": bool(cfg.get("fp8_weights", False)),
                   "decode_splits": splits, "input_replicas": R, "inputs": INPUT_NOTE},
        "roofline": {"bound": "hbm",
                     "kernel": ("mla_decode_latent_attn_packed" if packed else
                                "mla_decode_latent_attn") + " (split + merge launches)",
                     "achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": attn_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": work["attn_bytes"],
                     "avg_launch_us": decode_ms * 1e3},
        "step": {"roofline_us": t_roof_step * 1e6, "frac_of_roofline": t_roof_step / (ms_step * 1e-3),
                 "bytes": work["step_bytes"], "flops": work["step_flops"],
                 "GB_s": work["step_bytes"] / (ms_step * 1e-3) / 1e9,
                 "TFLOP_s": work["step_flops"] / (ms_step * 1e-3) / 1e12,
                 "launch": ("eager" if args.no_graph else
                            f"hip_graph_replay ({G} steps per graph, cycling over {R} input replicas)"),
                 "path": ("three calls: mla_absorb_q, mla_decode_latent_attn, mla_out_up"
                          if args.three_calls else
                          "mla_decode_step: absorb, split attention, split merge fused into W^UV"),
                 "eager_step_us": eager_ms * 1e3,
                 "absorb_us": absorb_ms * 1e3, "decode_us": decode_ms * 1e3,
                 "out_up_us": outup_ms * 1e3},
        "published_baseline": "none: the source pages print no throughput figures",
        "step_stats": stats,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.config, inp)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
