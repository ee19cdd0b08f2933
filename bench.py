"""Benchmark of one SVG2-form sparse attention layer on one MI355X.

Workload (default): the 5 s clip layer -- 32,760 latent tokens (21x30x52 grid)
x 40 heads, d=128, bf16; k-means with C_q=100 / C_k=500 for 10 iterations,
top-p 0.9; seeded synthetic mixture-of-Gaussians tokens (centre scale 1.75,
about 85% sparsity).  A step is one pass of the whole hot path: k-means of Q
and of K, the cluster sort of Q and of K (the Q side on a second stream,
concurrently with the K side), top-p selection, block-sparse attention that
reads Q/K/V through the permutation and writes O in token order (``--unfused``:
gather the permuted Q/K/V, attend, unpermute O).  Inputs are resident in HBM
before timing.

Prints one JSON line: value = effective TFLOP/s of the layer (4 d x kept
(query, key) pairs per step / step time), ms_per_step = ms per layer, plus the
per-stage breakdown, dense attention on the same tensors, the attention
kernel's roofline and the fp64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "ms/layer + effective TFLOP/s (frac of bf16 MFMA peak), 32,760 tok x 40 heads"
ATTN_SRC = os.path.join(ROOT, "sparse_attention_long_head_amd", "csrc", "attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_5s_traffic.txt")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def attention_traffic():
    """HBM bytes per attention launch from the committed counter summary, or None if
    the summary is missing or was taken on a different attention kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line)
        src = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
        if kv.get("attention_source_sha256", "").strip() != src:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(cfg, heads=(0, 1, 2, 3, 4, 5)):
    """The fp64 oracle's whole layer on a few heads (same tensors, same seeds); about
    10-20 s of host time at the 5 s clip size."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info()) or 1
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    x = synth.video_qkv(cfg, heads=heads)
    iq = synth.kmeans_init_indices(cfg, "q", cfg.cq, heads=heads)
    ik = synth.kmeans_init_indices(cfg, "k", cfg.ck, heads=heads)
    scale = float(np.float32(1.0 / np.sqrt(cfg.d)))
    flops = 0.0
    t0 = time.perf_counter()
    for j in range(len(heads)):
        q, k, v = (x[n][0, j].astype(np.float64) for n in "qkv")
        r = oracle.svg2_layer(q, k, v, q[iq[0, j]], k[ik[0, j]], cfg.iters, cfg.top_p, scale)
        flops += 4.0 * cfg.d * r["kept_pairs"]
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(heads)} of {cfg.heads} heads, whole layer (k-means x2, select, "
                      f"masked attention) in fp64 NumPy; {dt:.1f} s; "
                      f"{dt / len(heads) * cfg.heads * 1e3:.0f} ms/layer extrapolated"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="5s", choices=["5s", "10s", "30s"])
    ap.add_argument("--top-p", type=float, default=None)
    ap.add_argument("--workload", default="svg2",
                    choices=["svg2", "static-mask", "static-ratio", "dynamic-threshold",
                             "kmeans-warm", "sweep", "adaptive"],
                    help="svg2: k-means clusters + top-p (the default); static-mask: the fixed "
                         "radial + random block mask at --static-sparsity, attention alone; "
                         "static-ratio / "
                         "dynamic-threshold: DynamicRad's two modes on uniform 128-token blocks; "
                         "kmeans-warm: the svg2 layer over a drifting denoising sequence with the "
                         "centroid cache (warm-started k-means)")
    ap.add_argument("--sweep-p", default="0.8,0.9,0.95")
    ap.add_argument("--sweep-alpha", default="1.5,1.75,2.0")
    ap.add_argument("--denoise-steps", type=int, default=4)
    ap.add_argument("--step-drift", type=float, default=0.05)
    ap.add_argument("--warm-iters", type=int, default=2,
                    help="kmeans-warm: Lloyd iterations of a warm-started call")
    ap.add_argument("--theta", type=float, default=None,
                    help="svg2: global threshold on centroid logits instead of top-p; "
                         "dynamic-threshold: threshold on block-mean logits (default 0)")
    ap.add_argument("--ratios", default="1,0.75,0.5",
                    help="static-ratio: kept share of the radial candidates per temporal distance")
    ap.add_argument("--static-sparsity", type=float, default=0.8,
                    help="static-mask: share of the 128x128 tiles left out (0.8 = 13,107 of "
                         "65,536 tiles kept; 0.85 = 9,830)")
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-static", action="store_true",
                    help="svg2 workload: skip the static-mask section (80%% and 85%% "
                         "sparsity, dense on the same tensors)")
    ap.add_argument("--unfused", action="store_true",
                    help="materialise the permuted Q/K/V and unpermute O (instead of reading "
                         "and writing through the permutation inside attention)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run 3 identity-permutation copies of Q (335.5 MB read + "
                         "335.5 MB written at 5 s) to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path runs on a single GPU (every stage "
              "is independent per head, so heads would shard across GPUs with no exchange).  "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import synth
    from sparse_attention_long_head_amd import SparseVideoAttention, sva_full_attn

    if args.workload == "kmeans-warm":
        return bench_kmeans_warm(args)
    if args.workload == "sweep":
        return bench_sweep(args)
    if args.workload == "static-mask":
        return bench_static_mask(args)
    if args.workload == "adaptive":
        return bench_adaptive(args)
    if args.workload != "svg2":
        return bench_dynamicrad(args)
    cfg = synth.CONFIGS[args.config]
    if args.top_p is not None:
        cfg = cfg.with_(top_p=args.top_p)
    dev = torch.device("cuda:0")
    log(f"[bench] generating {cfg.name}: {cfg.n} tokens x {cfg.heads} heads, d={cfg.d}")
    x = synth.video_qkv(cfg)
    init_q = synth.gather_init(x["q"], synth.kmeans_init_indices(cfg, "q", cfg.cq))
    init_k = synth.gather_init(x["k"], synth.kmeans_init_indices(cfg, "k", cfg.ck))
    t = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in "qkv"}
    iq = torch.from_numpy(init_q).to(dev)
    ik = torch.from_numpy(init_k).to(dev)
    del x
    layer = SparseVideoAttention(cfg.batch, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck, cfg.iters,
                                 cfg.top_p, device=dev, fuse_permutation=not args.unfused,
                                 theta=args.theta)
    # "cluster" = k-means + permutation of Q (side stream) and of K/V, joined
    stages = ("cluster", "select", "attention", "unpermute")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        layer.cluster(t["q"], t["k"], t["v"], iq, ik)
        if ev is not None:
            ev[1].record()
        layer.select()
        if ev is not None:
            ev[2].record()
        layer.attend(t["q"], t["k"], t["v"])
        if ev is not None:
            ev[3].record()
        layer.unpermute()
        if ev is not None:
            ev[4].record()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kept = layer.kept_pairs()
    density = kept / float(cfg.batch * cfg.heads * cfg.n * cfg.n)
    flops = 4.0 * cfg.d * kept

    log(f"[bench] timing {args.steps} steps")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    per_stage = {name: statistics.median(events[s][i].elapsed_time(events[s][i + 1])
                                         for s in range(args.steps))
                 for i, name in enumerate(stages)}
    ia = stages.index("attention")
    attn_ms = statistics.mean(events[s][ia].elapsed_time(events[s][ia + 1]) for s in range(args.steps))
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12

    dense = None
    if not args.no_dense:
        log("[bench] dense attention on the same tensors")
        o = torch.empty_like(t["q"])
        sva_full_attn(t["q"], t["k"], t["v"], layer.scale, o=o)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.dense_reps):
            sva_full_attn(t["q"], t["k"], t["v"], layer.scale, o=o)
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.dense_reps
        dense_flops = 4.0 * cfg.d * cfg.batch * cfg.heads * cfg.n * cfg.n
        dense = {"ms": dense_ms, "tflops": dense_flops / (dense_ms * 1e-3) / 1e12,
                 "frac_of_peak": dense_flops / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                 "speedup_attention_only": dense_ms / attn_ms,
                 "speedup_whole_layer": dense_ms / ms_step}

    stage_roof = stage_rooflines(layer, t, iq, ik, cfg)
    static = None if (args.no_static or args.config != "5s") else static_mask_summary(args)

    if args.copy_calibration:
        from sparse_attention_long_head_amd import sva_unpermute
        ident = torch.arange(cfg.n, dtype=torch.int32, device=dev).repeat(
            cfg.batch * cfg.heads).reshape(cfg.batch, cfg.heads, cfg.n).contiguous()
        dst = torch.empty_like(t["q"])
        for _ in range(3):
            sva_unpermute(t["q"], ident, dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x {t['q'].numel() * 2 / 1e6:.1f} MB read + written")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] fp64 oracle on a bounded sample (host cores)")
        cpu = cpu_baseline(cfg)

    value = flops / (ms_step * 1e-3) / 1e12
    traffic = attention_traffic()
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded mixture-of-Gaussians video tokens (no dataset)",
        "config": {"workload": f"svg2 sparse attention layer, {cfg.name} clip",
                   "tokens": cfg.n, "grid_thw": [cfg.T, cfg.H, cfg.W], "heads": cfg.heads,
                   "head_dim": cfg.d, "batch": cfg.batch, "cq": cfg.cq, "ck": cfg.ck,
                   "kmeans_iters": cfg.iters, "top_p": cfg.top_p, "theta": args.theta,
                   "fused_permutation": not args.unfused, "centre_scale": cfg.alpha,
                   "density": round(density, 5), "kept_pairs": kept},
        "ms_per_layer": round(ms_step, 4),
        "frac_of_peak_layer": round(value / PEAK_BF16_TFLOPS, 5),
        "stages_ms_median": {k: round(v, 4) for k, v in per_stage.items()},
        "attention": {"ms": round(attn_ms, 4), "effective_tflops": round(attn_tflops, 2),
                      "frac_of_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4)},
        "dense": None if dense is None else {k: round(v, 4) for k, v in dense.items()},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "stage_rooflines": stage_roof,
        "static_mask": static,
    }
    print(json.dumps(out), flush=True)
    return 0


def static_mask_summary(args, sparsities=(0.8, 0.85), steps=5, warmup=2):
    """The static-mask configuration timed inside the default run: i.i.d. N(0,1)
    Q/K/V at the 5 s clip size, the radial candidate set padded with seeded
    random tiles to exactly each sparsity (uniform 128-token blocks), block-sparse
    attention alone, and dense attention on the same tensors for the speed-up."""
    import torch

    import synth
    from sparse_attention_long_head_amd import lib, sva_block_sparse_attn, sva_full_attn

    cfg = synth.CONFIGS["static"]
    dev = torch.device("cuda:0")
    log(f"[bench] static mask: {cfg.n} tokens x {cfg.heads} heads, sparsity {sparsities}")
    x = synth.video_qkv(cfg)
    t = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in "qkv"}
    del x
    bh = cfg.batch * cfg.heads
    scale = float(np.float32(1.0 / np.sqrt(cfg.d)))
    sizes = np.diff(synth.uniform_offsets(cfg.n, cfg.block)).astype(np.int64)
    o = torch.empty_like(t["q"])
    out = {"workload": f"static radial + random block mask, uniform {cfg.block}-token blocks, "
                       "i.i.d. N(0,1) Q/K/V, block-sparse attention alone",
           "tokens": cfg.n, "heads": cfg.heads, "head_dim": cfg.d}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    dense_ms = timed(lambda: sva_full_attn(t["q"], t["k"], t["v"], scale, o=o), args.dense_reps)
    dflops = 4.0 * cfg.d * bh * cfg.n * cfg.n
    out["dense"] = {"ms": round(dense_ms, 4),
                    "frac_of_peak": round(dflops / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    for sp in sparsities:
        mask = synth.static_block_mask(cfg, sp)
        count, idx = synth.mask_to_ell(mask)
        nb = mask.shape[0]
        off = torch.from_numpy(synth.uniform_offsets(cfg.n, cfg.block)).to(dev)
        off = off.expand(cfg.batch, cfg.heads, nb + 1).contiguous()
        kc = torch.from_numpy(count).to(dev).expand(cfg.batch, cfg.heads, nb).contiguous()
        ki = torch.from_numpy(idx).to(dev).expand(cfg.batch, cfg.heads, nb, nb).contiguous()
        ws = torch.empty(max(lib().sva_attn_workspace_bytes(cfg.batch, cfg.heads, cfg.n, nb), 1),
                         dtype=torch.uint8, device=dev)
        run = lambda: sva_block_sparse_attn(t["q"], t["k"], t["v"], off, off, kc, ki, scale,
                                            o=o, ws=ws)
        for _ in range(warmup):
            run()
        ms = timed(run, steps)
        kept = int(sizes @ mask.astype(np.int64) @ sizes) * bh
        tf = 4.0 * cfg.d * kept / (ms * 1e-3) / 1e12
        out[f"sparsity_{sp:.2f}"] = {
            "kept_tiles": int(mask.sum()), "tiles": int(nb * nb),
            "density": round(kept / float(bh * cfg.n * cfg.n), 5), "ms": round(ms, 4),
            "effective_tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "speedup_over_dense": round(dense_ms / ms, 3)}
    return out


def stage_rooflines(layer, t, iq, ik, cfg, reps=3):
    """The layer's other stages timed alone (after the timed steps, same buffers,
    events on the launch stream), each against the roofline that bounds it:
    k-means (2 n C d FLOP per iteration on MFMA; its minimum HBM traffic is X read
    twice per iteration, by the assignment and the mean), the cluster sort (4 B
    read + 4 B written per row, plus the offsets), the top-p selection (the
    centroids and sizes read, the mask and kept lists written)."""
    import torch

    from sparse_attention_long_head_amd import sva_kmeans, sva_permute, sva_select_blocks

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    bh, n, d = cfg.batch * cfg.heads, cfg.n, cfg.d
    out = {}
    for name, x, init, c, cent, asg, sz in (("kmeans_q", t["q"], iq, cfg.cq, layer.cent_q,
                                             layer.assign_q, layer.sizes_q),
                                            ("kmeans_k", t["k"], ik, cfg.ck, layer.cent_k,
                                             layer.assign_k, layer.sizes_k)):
        def run():
            cent.copy_(init)
            sva_kmeans(x, c, cfg.iters, cent, asg, sz, ws=layer.ws)
        ms = timed(run)
        flops = 2.0 * bh * n * c * d * cfg.iters
        hbm = 2.0 * cfg.iters * bh * n * d * 2
        out[name] = {"ms": round(ms, 4), "clusters": c, "iters": cfg.iters,
                     "algorithmic_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "min_hbm_gbs": round(hbm / (ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(hbm / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    for name, asg, c, perm, off in (("sort_q", layer.assign_q, cfg.cq, layer.perm_q, layer.off_q),
                                    ("sort_k", layer.assign_k, cfg.ck, layer.perm_k, layer.off_k)):
        ms = timed(lambda: sva_permute(asg, c, [], perm, off, ws=layer.ws))
        nbytes = bh * (8.0 * n + 4.0 * (c + 1))
        out[name] = {"ms": round(ms, 4), "algorithmic_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 5)}
    ms = timed(lambda: sva_select_blocks(layer.cent_q, layer.sizes_q, layer.cent_k, layer.sizes_k,
                                         layer.scale, layer.top_p, layer.mask, layer.kept_count,
                                         layer.kept_idx))
    nbytes = bh * (4.0 * (cfg.cq + cfg.ck) * (d + 1) + cfg.cq * cfg.ck * (1 + 4) + 4.0 * cfg.cq)
    out["select"] = {"ms": round(ms, 4), "algorithmic_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 5),
                     "bound": "latency (a few kilobytes per slice, sorted per Q cluster)"}
    return out


def _timed(stages, step, steps, warmup):
    """Run warmup + timed steps with per-stage events; returns (ms/step, per-stage medians)."""
    import torch
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step(events[s])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    per = {name: statistics.median(events[s][i].elapsed_time(events[s][i + 1])
                                   for s in range(steps)) for i, name in enumerate(stages)}
    return ms, per, events


def cpu_baseline_dynamicrad(cfg, x, workload, ratios, theta, heads=tuple(range(8))):
    """The fp64 oracle on a bounded sample (a few heads of the same tensors):
    each head's mask, then its masked attention; about 5-10 s of host time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info()) or 1
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    hw = cfg.H * cfg.W
    scale = float(np.float32(1.0 / np.sqrt(cfg.d)))
    rows = np.arange(cfg.n)
    flops = 0.0
    t0 = time.perf_counter()
    for h in heads:
        q, k, v = (x[n][0, h].astype(np.float64) for n in "qkv")
        if workload == "static-ratio":
            mask = oracle.static_ratio_mask(cfg.n, hw, cfg.block, 2, 8, ratios)
        else:
            cand = oracle.radial_candidates(cfg.n, hw, cfg.block, 2, 8)
            mq, sq = oracle.block_means(q, cfg.block)
            mk, sk = oracle.block_means(k, cfg.block)
            mask = oracle.threshold_select(oracle.centroid_scores(mq, mk, scale), sq, sk, theta,
                                           cand).mask
        oracle.block_sparse_attention(q, k, v, mask, cfg.block, scale, rows=rows)
        sizes = np.diff(np.minimum(np.arange(mask.shape[0] + 1) * cfg.block, cfg.n))
        flops += 4.0 * cfg.d * float((mask[rows // cfg.block] * sizes[None, :]).sum())
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(heads)} of {cfg.heads} heads: mask, then masked attention of all "
                      f"{cfg.n} query rows in fp64 NumPy; {dt:.1f} s"}


def cpu_baseline_static(cfg, x, mask, heads=(0, 1, 2, 3)):
    """The fp64 oracle's masked attention on a few heads of the same tensors (all
    query rows); about 10-20 s of host time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info()) or 1
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    scale = float(np.float32(1.0 / np.sqrt(cfg.d)))
    sizes = np.diff(synth_offsets(cfg)).astype(np.float64)
    pairs = float(sizes @ mask.astype(np.float64) @ sizes)
    t0 = time.perf_counter()
    for h in heads:
        q, k, v = (x[n][0, h].astype(np.float64) for n in "qkv")
        oracle.block_sparse_attention(q, k, v, mask, cfg.block, scale)
    dt = time.perf_counter() - t0
    flops = 4.0 * cfg.d * pairs * len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(heads)} of {cfg.heads} heads, masked attention of all {cfg.n} "
                      f"query rows in fp64 NumPy; {dt:.1f} s"}


def synth_offsets(cfg):
    import synth
    return synth.uniform_offsets(cfg.n, cfg.block)


def bench_static_mask(args) -> int:
    """The static-mask configuration: i.i.d. N(0,1) Q/K/V at the 5 s clip size
    and the radial candidate set padded with seeded random tiles to exactly the
    requested sparsity, one mask for all heads, uniform 128-token blocks in
    token order.  A step is sva_block_sparse_attn alone (the mask is an input
    built outside the timed region); dense attention on the same tensors is the
    reference for the speed-up."""
    import torch

    import synth
    from sparse_attention_long_head_amd import sva_block_sparse_attn, sva_full_attn, lib

    cfg = synth.CONFIGS["static"]
    sp = args.static_sparsity
    dev = torch.device("cuda:0")
    log(f"[bench] static-mask: {cfg.n} tokens x {cfg.heads} heads, sparsity {sp}")
    x = synth.video_qkv(cfg)
    mask = synth.static_block_mask(cfg, sp)
    count, idx = synth.mask_to_ell(mask)
    nb = mask.shape[0]
    bh = cfg.batch * cfg.heads
    t = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in "qkv"}
    off = torch.from_numpy(synth.uniform_offsets(cfg.n, cfg.block)).to(dev)
    off = off.expand(cfg.batch, cfg.heads, nb + 1).contiguous()
    kc = torch.from_numpy(count).to(dev).expand(cfg.batch, cfg.heads, nb).contiguous()
    ki = torch.from_numpy(idx).to(dev).expand(cfg.batch, cfg.heads, nb, nb).contiguous()
    scale = float(np.float32(1.0 / np.sqrt(cfg.d)))
    o = torch.empty_like(t["q"])
    ws = torch.empty(max(lib().sva_attn_workspace_bytes(cfg.batch, cfg.heads, cfg.n, nb), 1),
                     dtype=torch.uint8, device=dev)
    stages = ("attention",)

    def step(ev):
        if ev is not None:
            ev[0].record()
        sva_block_sparse_attn(t["q"], t["k"], t["v"], off, off, kc, ki, scale, o=o, ws=ws)
        if ev is not None:
            ev[1].record()

    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    ms, per, events = _timed(stages, step, args.steps, args.warmup)
    sizes = np.diff(synth.uniform_offsets(cfg.n, cfg.block)).astype(np.int64)
    kept = int(sizes @ mask.astype(np.int64) @ sizes) * bh
    flops = 4.0 * cfg.d * kept
    attn_ms = statistics.mean(events[s][0].elapsed_time(events[s][1]) for s in range(args.steps))
    attn_tf = flops / (attn_ms * 1e-3) / 1e12
    dense = None
    if not args.no_dense:
        log("[bench] dense attention on the same tensors")
        od = torch.empty_like(t["q"])
        sva_full_attn(t["q"], t["k"], t["v"], scale, o=od)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.dense_reps):
            sva_full_attn(t["q"], t["k"], t["v"], scale, o=od)
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.dense_reps
        dflops = 4.0 * cfg.d * bh * cfg.n * cfg.n
        dense = {"ms": dense_ms, "tflops": dflops / (dense_ms * 1e-3) / 1e12,
                 "frac_of_peak": dflops / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                 "speedup_attention_only": dense_ms / attn_ms}
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] fp64 oracle on a bounded sample (host cores)")
        cpu = cpu_baseline_static(cfg, x, mask)
    value = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) tokens and a seeded static block mask "
                "(no dataset)",
        "config": {"workload": f"static radial + random block mask at {sp:.0%} sparsity, "
                               f"uniform {cfg.block}-token blocks, attention alone",
                   "tokens": cfg.n, "grid_thw": [cfg.T, cfg.H, cfg.W], "heads": cfg.heads,
                   "head_dim": cfg.d, "block": cfg.block, "kept_tiles": int(mask.sum()),
                   "tiles": int(nb * nb), "sparsity_tiles": round(1 - mask.sum() / nb / nb, 5),
                   "density": round(kept / float(bh * cfg.n * cfg.n), 5), "kept_pairs": kept},
        "ms_per_layer": round(ms, 4),
        "stages_ms_median": {k: round(v_, 4) for k, v_ in per.items()},
        "attention": {"ms": round(attn_ms, 4), "effective_tflops": round(attn_tf, 2),
                      "frac_of_peak": round(attn_tf / PEAK_BF16_TFLOPS, 4)},
        "dense": None if dense is None else {k: round(v_, 4) for k, v_ in dense.items()},
        "roofline": {"bound": "mfma", "achieved": round(attn_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_adaptive(args) -> int:
    """The layer with a cluster count per head: C_q and C_k chosen per head by
    choose_clusters (ladders C/2, C, 2C around the clip's counts; the smallest
    whose k-means objective is within 10% of the objective at the largest),
    then the layer timed with those counts (heads with equal counts run as one
    group).  The calibration is outside the timed steps."""
    import torch

    import synth
    from sparse_attention_long_head_amd import (AdaptiveSparseVideoAttention, choose_clusters,
                                                strided_rows)

    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    log(f"[bench] adaptive: generating {cfg.name}")
    x = synth.video_qkv(cfg)
    t = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in "qkv"}
    del x
    lq = (cfg.cq // 2, cfg.cq, 2 * cfg.cq)
    lk = (cfg.ck // 2, cfg.ck, 2 * cfg.ck)
    t0 = time.perf_counter()
    cq, rq = choose_clusters(t["q"], lq, iters=5)
    ck, rk = choose_clusters(t["k"], lk, iters=5)
    calib_s = time.perf_counter() - t0
    layer = AdaptiveSparseVideoAttention(cfg.heads, cfg.n, cfg.d, cq, ck, cfg.iters, cfg.top_p,
                                         device=dev)
    inits = [(strided_rows(t["q"][:, hs], g.cq), strided_rows(t["k"][:, hs], g.ck))
             for hs, g in layer.groups]
    iq, ik = [a for a, _ in inits], [b for _, b in inits]
    stages = ("layer",)

    def step(ev):
        if ev is not None:
            ev[0].record()
        layer(t["q"], t["k"], t["v"], iq, ik)
        if ev is not None:
            ev[1].record()

    ms, per, _ = _timed(stages, step, args.steps, args.warmup)
    kept = layer.kept_pairs()
    flops = 4.0 * cfg.d * kept
    value = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded mixture-of-Gaussians video tokens (no dataset)",
        "config": {"workload": f"svg2 layer with per-head cluster counts, {cfg.name} clip",
                   "tokens": cfg.n, "heads": cfg.heads, "head_dim": cfg.d,
                   "ladder_q": list(lq), "ladder_k": list(lk), "cq_per_head": cq,
                   "ck_per_head": ck, "groups": len(layer.groups),
                   "density": round(kept / float(cfg.heads * cfg.n * cfg.n), 5),
                   "calibration_s": round(calib_s, 2)},
        "objective_over_scatter_q": np.round(rq, 5).tolist(),
        "objective_over_scatter_k": np.round(rk, 5).tolist(),
        "ms_per_layer": round(ms, 4),
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_dynamicrad(args) -> int:
    """DynamicRad's static-ratio or dynamic-threshold mode on uniform 128-token
    blocks at the 5 s clip size; one step = (block means + threshold, dynamic
    only) + block-sparse attention.  The static mask depends on geometry only
    and is built once, outside the timed steps."""
    import torch

    import synth
    from sparse_attention_long_head_amd import RadialSparseAttention

    static = args.workload == "static-ratio"
    # static: config 2's i.i.d. N(0,1) tensors; dynamic: the 5 s mixture tokens
    cfg = synth.CONFIGS["static" if static else "5s"]
    ratios = [float(r) for r in args.ratios.split(",")]
    theta = 0.0 if args.theta is None else args.theta
    dev = torch.device("cuda:0")
    log(f"[bench] {args.workload}: generating {cfg.name}: {cfg.n} tokens x {cfg.heads} heads")
    x = synth.video_qkv(cfg)
    t = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in "qkv"}
    layer = RadialSparseAttention(cfg.batch, cfg.heads, cfg.n, cfg.d, cfg.H * cfg.W, cfg.block,
                                  "static" if static else "dynamic", ratios=ratios,
                                  dt_max=len(ratios) - 1, theta=theta, device=dev)
    stages = ("select", "attention")

    def step(ev):
        if ev is not None:
            ev[0].record()
        layer.select(t["q"], t["k"])
        if ev is not None:
            ev[1].record()
        layer.attend(t["q"], t["k"], t["v"])
        if ev is not None:
            ev[2].record()

    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    ms, per, events = _timed(stages, step, args.steps, args.warmup)
    kept = layer.kept_pairs()
    flops = 4.0 * cfg.d * kept
    attn_ms = statistics.mean(events[s][1].elapsed_time(events[s][2]) for s in range(args.steps))
    attn_tf = flops / (attn_ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] fp64 oracle on a bounded sample (host cores)")
        cpu = cpu_baseline_dynamicrad(cfg, x, args.workload, ratios, theta)
    value = flops / (ms * 1e-3) / 1e12
    density = kept / float(cfg.batch * cfg.heads * cfg.n * cfg.n)
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded video tokens (no dataset)",
        "config": {"workload": f"dynamicrad {args.workload} on uniform {cfg.block}-token blocks, "
                               f"5s clip geometry", "tokens": cfg.n,
                   "grid_thw": [cfg.T, cfg.H, cfg.W], "heads": cfg.heads, "head_dim": cfg.d,
                   "block": cfg.block, "dt_max": len(ratios) - 1, "window0": 8,
                   "ratios": ratios if static else None, "theta": None if static else theta,
                   "density": round(density, 5), "kept_pairs": kept},
        "ms_per_layer": round(ms, 4),
        "stages_ms_median": {k: round(v, 4) for k, v in per.items()},
        "attention": {"ms": round(attn_ms, 4), "effective_tflops": round(attn_tf, 2),
                      "frac_of_peak": round(attn_tf / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_sweep(args) -> int:
    """Density / error / time over top-p x centre scale alpha (the content's
    cluster separation) on one clip config: for every alpha the clip is drawn
    anew and dense attention is the reference; for every p the whole layer is
    timed and its output compared with dense (relative L2 error over all heads,
    both bf16 outputs of this library)."""
    import torch

    import synth
    from sparse_attention_long_head_amd import SparseVideoAttention, sva_full_attn

    base = synth.CONFIGS[args.config]
    ps = [float(v) for v in args.sweep_p.split(",")]
    alphas = [float(v) for v in args.sweep_alpha.split(",")]
    dev = torch.device("cuda:0")
    rows = []
    dense_ms = None
    for alpha in alphas:
        cfg = base.with_(alpha=alpha)
        log(f"[bench] sweep {cfg.name}: alpha {alpha}: generating {cfg.n} x {cfg.heads}")
        x = synth.video_qkv(cfg)
        iq = torch.from_numpy(synth.gather_init(x["q"], synth.kmeans_init_indices(cfg, "q", cfg.cq))).to(dev)
        ik = torch.from_numpy(synth.gather_init(x["k"], synth.kmeans_init_indices(cfg, "k", cfg.ck))).to(dev)
        t = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in "qkv"}
        del x
        layer = SparseVideoAttention(cfg.batch, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck,
                                     cfg.iters, ps[0], device=dev)
        o_dense = torch.empty_like(t["q"])
        sva_full_attn(t["q"], t["k"], t["v"], layer.scale, o=o_dense)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sva_full_attn(t["q"], t["k"], t["v"], layer.scale, o=o_dense)
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1)
        dn = float(o_dense.float().norm())
        for p in ps:
            layer.top_p = p
            stages = ("cluster", "select", "attention")

            def step(ev):
                if ev is not None:
                    ev[0].record()
                layer.cluster(t["q"], t["k"], t["v"], iq, ik)
                if ev is not None:
                    ev[1].record()
                layer.select()
                if ev is not None:
                    ev[2].record()
                layer.attend(t["q"], t["k"], t["v"])
                if ev is not None:
                    ev[3].record()

            ms, per, _ = _timed(stages, step, max(2, min(args.steps, 5)), 1)
            kept = layer.kept_pairs()
            density = kept / float(cfg.batch * cfg.heads * cfg.n * cfg.n)
            err = float((layer.o.float() - o_dense.float()).norm()) / dn
            rows.append({"alpha": alpha, "top_p": p, "density": round(density, 5),
                         "ms_layer": round(ms, 3), "ms_attention": round(per["attention"], 3),
                         "ms_dense_attention": round(dense_ms, 3),
                         "speedup_attention": round(dense_ms / per["attention"], 3),
                         "speedup_layer": round(dense_ms / ms, 3),
                         "effective_tflops_attention":
                             round(4.0 * cfg.d * kept / (per["attention"] * 1e-3) / 1e12, 1),
                         "rel_l2_error_vs_dense": round(err, 5)})
            log(f"[bench]   p {p}: density {density:.4f}, layer {ms:.2f} ms, "
                f"attention {per['attention']:.2f} ms, rel err {err:.4f}")
        del layer, t, o_dense
        torch.cuda.empty_cache()
    out = {"metric": "density / error / time sweep over top-p x alpha", "config":
           {"workload": f"svg2 layer sweep, {base.name} clip", "tokens": base.n,
            "heads": base.heads, "cq": base.cq, "ck": base.ck, "kmeans_iters": base.iters},
           "data": "synthetic: seeded mixture-of-Gaussians video tokens (no dataset)",
           "rows": rows}
    print(json.dumps(out), flush=True)
    return 0


def _objective(x, cent, assign):
    """sum over rows of ||x - cent[assign]||^2 in fp64 (a measurement, not the path)."""
    import torch
    c = torch.gather(cent.double(), 2, assign.long()[..., None].expand(-1, -1, -1, cent.shape[-1]))
    return float(((x.double() - c) ** 2).sum())


def bench_kmeans_warm(args) -> int:
    """The centroid cache (Sparse VideoGen2, section 2.c).  Over a drifting
    denoising sequence X_s = X_0 + s * step_drift * Delta (5 s clip tensors),
    with the cache advanced the way the layer advances it (warm_iters
    iterations from the previous step's centroids): (1) at every step, the
    objective of 1..10 warm iterations relative to a cold 10-iteration run from
    the fixed initial rows, and the first count that reaches the cold
    objective; (2) the whole layer timed in warm mode with warm_iters."""
    import torch

    import synth
    from sparse_attention_long_head_amd import SparseVideoAttention, sva_kmeans

    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    S = max(1, args.denoise_steps)
    log(f"[bench] kmeans-warm: {cfg.name}, {S} denoising steps, step drift {args.step_drift}")
    x = synth.video_qkv(cfg)
    idx = {w: torch.from_numpy(synth.kmeans_init_indices(cfg, w, cfg.cq if w == "q" else cfg.ck))
           .to(dev) for w in "qk"}
    x0 = {n: torch.from_numpy(x[n]).to(dev) for n in "qkv"}
    delta = {w: torch.from_numpy(synth.denoise_direction(cfg, w)).to(dev) for w in "qk"}
    del x
    seq = [{w: (x0[w] + float(s * args.step_drift) * delta[w]).to(torch.bfloat16) for w in "qk"}
           for s in range(S + 1)]
    v = x0["v"].to(torch.bfloat16)
    del delta
    c_of = {"q": cfg.cq, "k": cfg.ck}

    def init_rows(xs, w):
        i = idx[w]
        return torch.gather(xs.float(), 2, i[..., None].expand(-1, -1, -1, cfg.d)).contiguous()

    from sparse_attention_long_head_amd import lib
    ws = torch.empty(lib().sva_kmeans_workspace_bytes(cfg.batch, cfg.heads, cfg.n, cfg.d,
                                                      max(c_of.values())),
                     dtype=torch.uint8, device=dev)
    asg = torch.empty(seq[0]["q"].shape[:3], dtype=torch.int32, device=dev)
    szs = {w: torch.empty(seq[0]["q"].shape[:2] + (c_of[w],), dtype=torch.int32, device=dev)
           for w in "qk"}

    def run(xs, w, cent, iters):
        sva_kmeans(xs, c_of[w], iters, cent, asg, szs[w], ws=ws)
        return asg

    def timed_ms(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    cache = {}
    for w in "qk":
        cache[w] = init_rows(seq[0][w], w)
        run(seq[0][w], w, cache[w], cfg.iters)
    rows = []
    for s in range(1, S + 1):
        row = {"step": s}
        for w in "qk":
            xs = seq[s][w]
            cent = init_rows(xs, w)
            a = run(xs, w, cent, cfg.iters)
            j_cold = _objective(xs, cent, a)
            cold_ms = timed_ms(lambda: run(xs, w, init_rows(xs, w), cfg.iters))
            need, ratio = None, []
            for it in range(1, cfg.iters + 1):
                cent_w = cache[w].clone()
                a = run(xs, w, cent_w, it)
                ratio.append(round(_objective(xs, cent_w, a) / j_cold, 6))
                if need is None and ratio[-1] <= 1.0:
                    need = it
            warm_ms = timed_ms(lambda: run(xs, w, cache[w].clone(), args.warm_iters))
            cent_w = cache[w].clone()
            run(xs, w, cent_w, args.warm_iters)
            cache[w] = cent_w
            row[w] = {"cold_objective": j_cold, "warm_over_cold_objective_by_iters": ratio,
                      "warm_iters_to_cold_objective": need, "cold_ms": round(cold_ms, 4),
                      "warm_ms": round(warm_ms, 4)}
        rows.append(row)
        log(f"[bench] step {s}: Q {row['q']['warm_iters_to_cold_objective']} it, "
            f"K {row['k']['warm_iters_to_cold_objective']} it")
    iters_warm = args.warm_iters

    # the layer in warm mode
    iq0, ik0 = init_rows(seq[0]["q"], "q"), init_rows(seq[0]["k"], "k")
    layer = SparseVideoAttention(cfg.batch, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck, cfg.iters,
                                 cfg.top_p, device=dev, iters_warm=iters_warm)
    layer(seq[0]["q"], seq[0]["k"], v, iq0, ik0)
    stages = ("cluster", "select", "attention")
    cur = [0]

    def step(ev):
        s = 1 + cur[0] % S
        cur[0] += 1
        if ev is not None:
            ev[0].record()
        layer.cluster(seq[s]["q"], seq[s]["k"], v)
        if ev is not None:
            ev[1].record()
        layer.select()
        if ev is not None:
            ev[2].record()
        layer.attend(seq[s]["q"], seq[s]["k"], v)
        if ev is not None:
            ev[3].record()

    ms, per, events = _timed(stages, step, args.steps, args.warmup)
    kept = layer.kept_pairs()
    flops = 4.0 * cfg.d * kept
    attn_ms = statistics.mean(events[s][2].elapsed_time(events[s][3]) for s in range(args.steps))
    attn_tf = flops / (attn_ms * 1e-3) / 1e12
    value = flops / (ms * 1e-3) / 1e12
    cold_km = sum(r[w]["cold_ms"] for r in rows for w in "qk") / S
    warm_km = sum(r[w]["warm_ms"] for r in rows for w in "qk") / S
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded mixture-of-Gaussians video tokens drifting over denoising "
                "steps (no dataset)",
        "config": {"workload": f"svg2 sparse attention layer with the centroid cache, {cfg.name} "
                               f"clip, {S}-step drifting sequence",
                   "tokens": cfg.n, "heads": cfg.heads, "head_dim": cfg.d, "cq": cfg.cq,
                   "ck": cfg.ck, "cold_iters": cfg.iters, "warm_iters": iters_warm,
                   "step_drift": args.step_drift, "top_p": cfg.top_p, "kept_pairs": kept},
        "ms_per_layer": round(ms, 4),
        "stages_ms_median": {k: round(v_, 4) for k, v_ in per.items()},
        "kmeans_ms_per_step": {"cold_q_plus_k": round(cold_km, 4),
                               "warm_q_plus_k": round(warm_km, 4),
                               "speedup": round(cold_km / warm_km, 3)},
        "convergence": rows,
        "attention": {"ms": round(attn_ms, 4), "effective_tflops": round(attn_tf, 2),
                      "frac_of_peak": round(attn_tf / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
