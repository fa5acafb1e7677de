#!/usr/bin/env python3
"""Throughput of the indexer hot path on one MI355X.

Workload (one "step"): one decode batch at L = 131072 -- 8 sequences, one query
each, H_I = 64 heads, d = 128, bf16 q / keys, fp32 w, k = 2048 -- pushed through
every selector of the library, with all inputs resident in HBM:
  1. DSA: score every causal prefix token with all heads, top-k; its key scan
     also writes the block means of the keys (HISA b = 128 and MISA B =
     1024), the pooling being done in the same pass over the key cache,
  2. MISA: router over the pooled keys, top-8 heads, routed scan, top-k
     (decode rows route inside the routed scan),
  3. MISA-dagger: routed top-k' (8192), rerank with all heads, top-k,
  4. HISA: block scores, top-64 blocks, exact rescoring of their 8192 tokens,
     top-k.
value = logical indexer scores per second = (query, legal token) pairs that the
four selectors rank per step / step time.

Also reported: per-kernel HIP-event durations inside the timed region, the
roofline fraction of the dominant kernel (the DSA decode scan, HBM-bound), the
fused causal prefill (T = 4096 new queries over 28672 cached keys, MFMA-bound)
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "indexer scores/s (query·token) + top-k rows/s at L=128K; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "sparse_attention_token_dsa_amd", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-iters", type=int, default=10)
    return ap.parse_args()


def source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_attention_token_dsa_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, digest):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    they were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("bytes_per_launch")


def measured_mfma(digest, key="prefill_fused_mfma"):
    """Counter-derived MFMA figures of the fused prefill (rocprofv3 --pmc,
    see traffic.py), or None if taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            e = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not e or e.get("source_digest") != digest:
        return None
    return {k: e[k] for k in ("mfma_busy_frac", "valu_per_mfma", "lds_bank_conflict_frac",
                              "active_cycles")}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the indexer shards by sequence with no communication); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_attention_token_dsa_amd import api, synth
    from sparse_attention_token_dsa_amd import workload as wl

    dev = torch.device("cuda:0")
    api.load()
    cfg = synth.CONFIGS["misa_128k_h64"]
    p = synth.make_config("misa_128k_h64")
    Bt, L, H, d, k = p["Bt"], p["L"], p["H"], p["d"], cfg["topk"]
    off = p["offset"]
    B, h, kp, b, r = 1024, 8, 8192, 128, 64
    q = torch.from_numpy(p["q"].view(np.int16)).to(dev)
    w = torch.from_numpy(p["w"]).to(dev)
    K = torch.from_numpy(p["K"].view(np.int16)).to(dev)

    # Preallocated outputs and workspaces: nothing is allocated in the loop.
    shape = api.Shape(Bt, 1, H, d, L, off, k)
    ws_dsa = torch.empty(api.indexer_score_topk_ws(shape), dtype=torch.uint8, device=dev)
    ws_m1 = torch.empty(api.misa_route_ws(shape, B, h, 0, True), dtype=torch.uint8, device=dev)
    ws_m2 = torch.empty(api.misa_route_ws(shape, B, h, kp, True), dtype=torch.uint8, device=dev)
    ws_hi = torch.empty(api.hisa_coarse_fine_ws(shape, b, r, True), dtype=torch.uint8,
                        device=dev)
    reps_b = torch.empty((Bt, L // b, 2, d), dtype=torch.int16, device=dev)
    reps_B = torch.empty((Bt, L // B, 2, d), dtype=torch.int16, device=dev)
    outs = {m: (torch.empty((Bt, 1, k), dtype=torch.int32, device=dev),
                torch.empty((Bt, 1, k), dtype=torch.float32, device=dev))
            for m in ("dsa", "misa", "misa_dagger", "hisa")}

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        # DSA, pooling the keys it streams into the b and B block means that
        # MISA and HISA read (one pass over the key cache for both)
        api.indexer_score_topk_pooled(q, w, K, off, k, b, B, out_small=reps_b, out_large=reps_B,
                                      out_idx=outs["dsa"][0], out_score=outs["dsa"][1],
                                      ws=ws_dsa)
        mark(1)
        api.misa_route(q, w, K, off, k, B, h, 0, pooled=reps_B, want_heads=False,
                       out_idx=outs["misa"][0], out_score=outs["misa"][1], ws=ws_m1)
        mark(2)
        api.misa_route(q, w, K, off, k, B, h, kp, pooled=reps_B, want_heads=False,
                       out_idx=outs["misa_dagger"][0], out_score=outs["misa_dagger"][1],
                       ws=ws_m2)
        mark(3)
        api.hisa_coarse_fine(q, w, K, off, k, b, r, reps=reps_b, want_blocks=False,
                             out_idx=outs["hisa"][0], out_score=outs["hisa"][1], ws=ws_hi)
        mark(4)

    # The same step on two streams (default priority).  The pooled DSA call
    # records an event as soon as the block means are written; HISA and then
    # MISA start on the second stream from it, while MISA-dagger (the longest
    # chain) follows DSA's top-k on the first.  Each cross-stream edge of a
    # HIP graph costs several microseconds, so the step uses just these two.
    side = torch.cuda.Stream(device=dev)
    pools_ready = torch.cuda.Event()
    pools_ready.record()  # created outside any capture

    def step_concurrent():
        main = torch.cuda.current_stream(dev)
        api.indexer_score_topk_pooled(q, w, K, off, k, b, B, out_small=reps_b, out_large=reps_B,
                                      out_idx=outs["dsa"][0], out_score=outs["dsa"][1],
                                      ws=ws_dsa, pools_ready=pools_ready)
        side.wait_event(pools_ready)
        with torch.cuda.stream(side):
            # HISA's latency-bound kernels first, beside DSA's top-k on the
            # first stream, then MISA's scan beside MISA-dagger's
            api.hisa_coarse_fine(q, w, K, off, k, b, r, reps=reps_b, want_blocks=False,
                                 out_idx=outs["hisa"][0], out_score=outs["hisa"][1], ws=ws_hi)
            api.misa_route(q, w, K, off, k, B, h, 0, pooled=reps_B, want_heads=False,
                           out_idx=outs["misa"][0], out_score=outs["misa"][1], ws=ws_m1)
        api.misa_route(q, w, K, off, k, B, h, kp, pooled=reps_B, want_heads=False,
                       out_idx=outs["misa_dagger"][0], out_score=outs["misa_dagger"][1],
                       ws=ws_m2)
        main.wait_stream(side)

    # The GPU's clocks ramp up over the first tens of milliseconds under load:
    # the step runs for SETTLE_S seconds before the warm-up steps proper.
    settle(lambda: step(), torch, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    # Eager pass: per-kernel HIP events recorded by the library on the launch
    # stream over exactly `steps` steps.
    api.profile_enable(True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    kern = api.profile_read()
    api.profile_enable(False)
    ms_eager = (t1 - t0) * 1e3 / args.steps

    # The step captured once into a HIP graph (no allocation, no memset nodes:
    # the library clears its state with a fill kernel), replayed for the
    # timed value.  Every replay of the check below must match the eager
    # result exactly (same kernels, same inputs).
    ref = {m: (o[0].clone(), o[1].clone()) for m, o in outs.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_concurrent()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize(dev)
        for m, o in outs.items():
            a_idx = torch.sort(o[0], -1)[0]
            r_idx = torch.sort(ref[m][0], -1)[0]
            if not torch.equal(a_idx, r_idx):
                raise RuntimeError("graph replay differs from the eager step (%s)" % m)
        step()  # eager work between replays
        torch.cuda.synchronize(dev)
    # Cold-cache timing.  The 256 MB infinity cache (MALL) in front of HBM
    # would otherwise still hold much of the 256 MiB key cache from the step
    # before.  Before every timed step a 1 GiB buffer is read (clean lines:
    # no write-back lands in the measured step), and each step is bracketed
    # by its own pair of events, so the flush is not timed.
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def flush():
        flush_buf.sum()

    for _ in range(args.warmup):
        flush()
        graph.replay()
    torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:
        flush()
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize(dev)
    ms_step = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps

    # Back to back, the cache warm from the step before (context only).
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    ms_step_warm = (t1 - t0) * 1e3 / args.steps

    # The DSA selector alone right after a flush: the dominant kernel's
    # roofline is taken on these launches.
    api.profile_enable(True)
    for _ in range(args.steps):
        flush()
        api.indexer_score_topk(q, w, K, off, k, *outs["dsa"], ws=ws_dsa)
    torch.cuda.synchronize(dev)
    kern_cold = api.profile_read()
    api.profile_enable(False)

    # Per-selector split (separate pass, torch events between the calls).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    split = {n: 0.0 for n in ("dsa_pool", "misa", "misa_dagger", "hisa")}
    nsplit = max(5, args.steps // 5)
    for _ in range(nsplit):
        step(ev)
        torch.cuda.synchronize(dev)
        for i, n in enumerate(split):
            split[n] += ev[i].elapsed_time(ev[i + 1]) / nsplit

    # Each selector alone, cache flushed before each call (pools given, as in
    # the step): the per-selector times behind the ratios and computed rates.
    sel_calls = {
        "dsa": lambda: api.indexer_score_topk(q, w, K, off, k, *outs["dsa"], ws=ws_dsa),
        "dsa_pool": lambda: api.indexer_score_topk_pooled(q, w, K, off, k, b, B, out_small=reps_b,
                                                          out_large=reps_B,
                                                          out_idx=outs["dsa"][0],
                                                          out_score=outs["dsa"][1], ws=ws_dsa),
        "misa": lambda: api.misa_route(q, w, K, off, k, B, h, 0, pooled=reps_B, want_heads=False,
                                       out_idx=outs["misa"][0], out_score=outs["misa"][1],
                                       ws=ws_m1),
        "misa_dagger": lambda: api.misa_route(q, w, K, off, k, B, h, kp, pooled=reps_B,
                                              want_heads=False, out_idx=outs["misa_dagger"][0],
                                              out_score=outs["misa_dagger"][1], ws=ws_m2),
        "hisa": lambda: api.hisa_coarse_fine(q, w, K, off, k, b, r, reps=reps_b,
                                             want_blocks=False, out_idx=outs["hisa"][0],
                                             out_score=outs["hisa"][1], ws=ws_hi),
    }
    sel_ms, sel_kern, sel_graph = {}, {}, {}
    for n, fn in sel_calls.items():
        sel_ms[n], kus = flushed_calls(api, torch, fn, flush, args.steps)
        sel_kern[n] = {x: round(v, 2) for x, v in kus.items()}
        sel_graph[n] = round(flushed_graph_ms(torch, fn, flush, args.steps), 4)

    rows = Bt  # one query per sequence
    pairs = wl.legal_pairs(1, off, batch=Bt)   # every legal token of each row
    logical_pairs = 4 * pairs                  # four selectors
    value = logical_pairs / (ms_step * 1e-3)
    kernels = {n: {"avg_us": 1e3 * t / c, "launches_per_step": c / args.steps}
               for n, (t, c) in sorted(kern.items())}
    computed = computed_work(rows, L, H, d, B, h, kp, b, r, pairs, sel_ms, ms_step)

    # Roofline of the DSA decode scan: algorithmic bytes per launch (the keys
    # once, q and w) over its average duration right after a cache flush (the
    # warm figure, from the eager step pass, for context).  The score rows
    # this design stages for its top-k are reported apart.
    kbytes = wl.key_bytes(Bt, L, d)
    scan_bytes = wl.scan_bytes(rows, Bt, L, H, d)
    design_bytes = wl.score_row_bytes(rows, L)
    scan_us = 1e3 * kern_cold["scan_dsa"][0] / kern_cold["scan_dsa"][1]
    scan_gbs = scan_bytes / (scan_us * 1e-6) / 1e9
    # (in the eager step the DSA scan is the pooled one)
    scan_us_warm = kernels["scan_dsa_pool"]["avg_us"]
    digest = source_digest(["scan.hip", "sa_frag.h", "sa_common.h"])
    roofline = {"kernel": "scan_dsa", "bound": "hbm", "achieved": round(scan_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(scan_gbs / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("scan_dsa", digest),
                "algorithmic_bytes_per_launch": scan_bytes,
                "design_bytes_per_launch": design_bytes,
                "design_bytes": "fp32 score rows written for the top-k (not in achieved)",
                "avg_us": round(scan_us, 2),
                "cache": "cold: a 1 GiB read before each launch",
                "avg_us_warm": round(scan_us_warm, 2),
                "warm_kernel": "scan_dsa_pool (the step's DSA scan, pooling the keys too)",
                "achieved_warm": round(scan_bytes / (scan_us_warm * 1e-6) / 1e9, 1)}
    pus = sel_kern["dsa_pool"]["scan_dsa_pool"]
    roofline["pooled_scan"] = {
        "kernel": "scan_dsa_pool", "cache": "cold", "avg_us": pus,
        "algorithmic_bytes_per_launch": scan_bytes + Bt * (L // b + L // B) * 4 * d,
        "frac": round((scan_bytes + Bt * (L // b + L // B) * 4 * d) / (pus * 1e-6) / 1e9
                      / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic("scan_dsa_pool", digest)}
    other_hbm = {}
    for name, nbytes in (("scan_routed", wl.scan_bytes(rows, Bt, L, h, d)),
                         ("scan_dsa_pool", wl.scan_bytes(rows, Bt, L, H, d)
                          + Bt * (L // b + L // B) * 4 * d)):
        if name in kernels:
            us = kernels[name]["avg_us"]
            gbs = nbytes / (us * 1e-6) / 1e9
            other_hbm[name] = {"cache": "warm", "avg_us": round(us, 2), "GB/s": round(gbs, 1),
                               "frac": round(gbs / HBM_PEAK_GBS, 4),
                               "algorithmic_bytes_per_launch": nbytes,
                               "traffic": measured_traffic(name, digest)}

    result = {
        "metric": METRIC, "value": value, "unit": "scores/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_128k_b8_h64", "batch": Bt, "L": L, "H_I": H, "d": d,
                   "topk": k, "misa": {"B": B, "h": h, "k_prime": kp},
                   "hisa": {"b": b, "r": r},
                   "step": "DSA with pooling (b=128, B=1024) in its key scan + MISA + "
                           "MISA-dagger + HISA"},
        "topk_rows_per_s": 4 * rows / (ms_step * 1e-3),
        "timing": "value and ms_per_step: the step replayed as one HIP graph: the pooled DSA "
                  "scan, then HISA and MISA on a second stream beside DSA's top-k and "
                  "MISA-dagger, each step after a 1 GiB read "
                  "that evicts the keys from the "
                  "256 MB infinity cache, timed with its own events; ms_per_step_warm: "
                  "back-to-back replays; ms_per_step_eager, the kernel table and "
                  "selector_ms: the step's calls one after another on one stream, with "
                  "HIP events",
        "ms_per_step_warm": ms_step_warm,
        "ms_per_step_eager": ms_eager,
        "selector_ms": {n: round(v, 4) for n, v in split.items()},
        "selector_ms_note": "selector_ms: eager step, one call after another, no flush "
                            "between them",
        "selector_ms_flushed": sel_ms,
        "selector_ms_flushed_graph": sel_graph,
        "selector_ms_flushed_note": "each call alone after a 1 GiB read: eager (the library's "
                                    "kernel events off), and captured alone into a HIP graph",
        "selector_kernels_us_flushed": sel_kern,
        "selector_scores_per_s": {n: pairs / (sel_ms[n] * 1e-3)
                                  for n in ("dsa", "misa", "misa_dagger", "hisa")},
        "computed": computed,
        "kernels": kernels,
        "roofline": roofline,
        "hbm_kernels": other_hbm,
    }

    result["decode_32k"] = bench_decode_32k(api, synth, torch, np, dev, flush, args.steps)
    result["h32"] = bench_h32(api, synth, torch, np, dev, flush, args.steps)
    result["ratios"] = {
        "what": "selector time ratios DSA / X on the same inputs, cache flushed before each "
                "call (pages' context, other hardware: MISA 3.82x, MISA-dagger 1.76x, "
                "HISA 4x at 128K)",
        "h64": {n: sel_ms["dsa"] / sel_ms[n] for n in ("misa", "misa_dagger", "hisa")},
        "h32": {n: result["h32"]["ms_per_call"]["dsa"] / v
                for n, v in result["h32"]["ms_per_call"].items() if n != "dsa"}}
    result["fp8"] = bench_fp8(api, torch, dev, q, w, K, shape, flush, args.steps)
    result["lisa"], result["resmisa"] = bench_lisa_resmisa(api, torch, dev, q, w, K, shape, flush,
                                                           args.steps)
    result["misa_hisa"] = bench_misa_hisa(api, torch, dev, q, w, K, shape, reps_b, reps_B, flush,
                                          args.steps)
    result["tidy"], result["ragged"] = bench_tidy_ragged(api, torch, dev, q, w, K, shape, outs,
                                                         flush, args.steps)

    if not args.no_prefill:
        result["prefill"] = bench_prefill(api, synth, torch, np, dev, args.prefill_iters)

    if not args.no_cpu_baseline:
        gpu_sets = {m: o[0].view(Bt, k).cpu().numpy() for m, o in outs.items()}
        result["cpu_baseline"], result["selection_margins"] = cpu_baseline(p, k, B, h, kp, b, r,
                                                                          gpu_sets)

    print(json.dumps(result))


SETTLE_S = 0.3


def settle(fn, torch, dev):
    """Run fn back to back for SETTLE_S seconds (at least twice), untimed."""
    t0 = time.perf_counter()
    n = 0
    while n < 2 or time.perf_counter() - t0 < SETTLE_S:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize(dev)
    torch.cuda.synchronize(dev)


def computed_work(rows, L, H, d, B, h, kp, b, r, pairs, split, ms_step):
    """(query, key) pairs each selector actually scores, and per-head dot
    products, per call and per second of the selector alone (split, cache
    flushed) and of the whole step."""
    nB, nb = -(-L // B), -(-L // b)
    sel = {
        "dsa": (pairs, pairs * H),
        "misa": (pairs + rows * nB, pairs * h + rows * nB * H),
        "misa_dagger": (pairs + rows * nB + rows * kp, pairs * h + rows * nB * H + rows * kp * H),
        "hisa": (rows * nb + rows * r * b, rows * nb * H + rows * r * b * H),
    }
    out = {"what": "pairs scored by each selector (any number of heads; MISA counts its "
                   "router's pooled keys, MISA-dagger its rerank, HISA its block "
                   "representatives and rescored tokens) and the per-head dot products "
                   "behind them; per_s uses the selector's own flushed time"}
    for n, (pc, dots) in sel.items():
        out[n] = {"pairs": pc, "dots": dots, "pairs_per_s": pc / (split[n] * 1e-3),
                  "dots_per_s": dots / (split[n] * 1e-3)}
    out["step_pairs_per_s"] = sum(v[0] for v in sel.values()) / (ms_step * 1e-3)
    out["step_dots_per_s"] = sum(v[1] for v in sel.values()) / (ms_step * 1e-3)
    return out


def bench_decode_32k(api, synth, torch, np, dev, flush, steps):
    """The DSA selector on the 32 x 32768 decode batch (64 heads, k = 2048),
    cache flushed before each call: scan time against the HBM roofline."""
    from sparse_attention_token_dsa_amd import workload as wl
    p = synth.make_config("decode_32k")
    q = torch.from_numpy(p["q"].view(np.int16)).to(dev)
    w = torch.from_numpy(p["w"]).to(dev)
    K = torch.from_numpy(p["K"].view(np.int16)).to(dev)
    Bt, L, H, d, off, k = p["Bt"], p["L"], p["H"], p["d"], p["offset"], 2048
    shape = api.Shape(Bt, 1, H, d, L, off, k)
    ws = torch.empty(api.indexer_score_topk_ws(shape), dtype=torch.uint8, device=dev)
    oi = torch.empty((Bt, 1, k), dtype=torch.int32, device=dev)
    osc = torch.empty((Bt, 1, k), dtype=torch.float32, device=dev)
    ms, kus = flushed_calls(api, torch, lambda: api.indexer_score_topk(q, w, K, off, k, oi, osc,
                                                                       ws=ws), flush, steps)
    nb = wl.scan_bytes(Bt, Bt, L, H, d)
    gbs = nb / (kus["scan_dsa"] * 1e-6) / 1e9
    pairs = wl.legal_pairs(1, off, batch=Bt)
    return {"workload": "decode_32k_b32_h64", "cache": "cold: a 1 GiB read before each call",
            "ms_per_call": ms, "scores_per_s": pairs / (ms * 1e-3),
            "topk_rows_per_s": Bt / (ms * 1e-3),
            "kernels_us": {n: round(v, 2) for n, v in kus.items()},
            "roofline": {"kernel": "scan_dsa", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "algorithmic_bytes_per_launch": nb,
                         "design_bytes_per_launch": wl.score_row_bytes(Bt, L),
                         "avg_us": round(kus["scan_dsa"], 2),
                         "target": "scan <= 48 us (70 % of 8 TB/s)"}}


def bench_h32(api, synth, torch, np, dev, flush, steps):
    """DSA, MISA (h = 8) and MISA-dagger (k' = 8192) on the 128K batch-8
    decode with 32 indexer heads (the GLM-5 indexer width), pooled keys given:
    per-call times after a cache flush."""
    p = synth.make_config("misa_128k_h32")
    q = torch.from_numpy(p["q"].view(np.int16)).to(dev)
    w = torch.from_numpy(p["w"]).to(dev)
    K = torch.from_numpy(p["K"].view(np.int16)).to(dev)
    Bt, L, H, d, off, k = p["Bt"], p["L"], p["H"], p["d"], p["offset"], 2048
    B, h, kp = 1024, 8, 8192
    shape = api.Shape(Bt, 1, H, d, L, off, k)
    pooled = api.pool_blocks(K, B)
    ws = torch.empty(max(api.indexer_score_topk_ws(shape), api.misa_route_ws(shape, B, h, kp, True)),
                     dtype=torch.uint8, device=dev)
    oi = torch.empty((Bt, 1, k), dtype=torch.int32, device=dev)
    osc = torch.empty((Bt, 1, k), dtype=torch.float32, device=dev)
    calls = {
        "dsa": lambda: api.indexer_score_topk(q, w, K, off, k, oi, osc, ws=ws),
        "misa": lambda: api.misa_route(q, w, K, off, k, B, h, 0, pooled=pooled, want_heads=False,
                                       out_idx=oi, out_score=osc, ws=ws),
        "misa_dagger": lambda: api.misa_route(q, w, K, off, k, B, h, kp, pooled=pooled,
                                              want_heads=False, out_idx=oi, out_score=osc, ws=ws),
    }
    ms, kern = {}, {}
    for n, fn in calls.items():
        ms[n], kus = flushed_calls(api, torch, fn, flush, steps)
        kern[n] = {x: round(v, 2) for x, v in kus.items()}
    return {"workload": "misa_128k_b8_h32", "cache": "cold: a 1 GiB read before each call",
            "config": {"B": B, "h": h, "k_prime": kp, "pooled": "given"},
            "ms_per_call": ms, "kernels_us": kern}


def bench_fp8(api, torch, dev, q, w, K, shape, flush, steps):
    """The DSA selector on the same decode batch with the keys held as E4M3
    codes plus one fp32 scale per key (132 B per key instead of 256 B)."""
    Bt, L, H, d, off, k = shape.batch, shape.L, shape.H, shape.d, shape.causal_offset, shape.topk
    codes = torch.empty((Bt, L, d), dtype=torch.uint8, device=dev)
    scales = torch.empty((Bt, L), dtype=torch.float32, device=dev)
    ws = torch.empty(api.indexer_score_topk_fp8_ws(shape), dtype=torch.uint8, device=dev)
    oi = torch.empty((Bt, 1, k), dtype=torch.int32, device=dev)
    osc = torch.empty((Bt, 1, k), dtype=torch.float32, device=dev)

    def call():
        api.indexer_score_topk_fp8(q, w, codes, scales, off, k, oi, osc, ws=ws)

    api.quantize_keys_fp8(K, codes, scales)
    settle(call, torch, dev)
    api.profile_enable(True)
    for _ in range(steps):
        flush()
        api.quantize_keys_fp8(K, codes, scales)
    torch.cuda.synchronize(dev)
    kq = api.profile_read()
    api.profile_enable(False)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    api.profile_enable(True)
    for e0, e1 in evs:
        flush()
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize(dev)
    kern = api.profile_read()
    api.profile_enable(False)
    ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps
    scan_bytes = Bt * L * (d + 4) + Bt * H * d * 2 + Bt * H * 4 + Bt * L * 4
    us = 1e3 * kern["scan_dsa_fp8"][0] / kern["scan_dsa_fp8"][1]
    gbs = scan_bytes / (us * 1e-6) / 1e9
    q_us = 1e3 * kq["quantize_fp8"][0] / kq["quantize_fp8"][1]
    q_bytes = Bt * L * (2 * d + d + 4)
    scan8_digest = source_digest(["scan8.hip", "sa_frag.h", "sa_common.h"])

    # The same selector with the query converted to E4M3 in the kernel and the
    # dot products on the fp8 MFMA (same bytes, a quarter of the MFMAs).
    def call_q():
        api.indexer_score_topk_fp8q(q, w, codes, scales, off, k, oi, osc, ws=ws)

    ms_q, kern_q = flushed_calls(api, torch, call_q, flush, steps)
    us_q = kern_q["scan_dsa_fp8q"]
    gbs_q = scan_bytes / (us_q * 1e-6) / 1e9

    # MISA (B 1024, h 8), MISA-dagger (k' 8192) and HISA (b 128, r 64) on the
    # same FP8 cache, block means given as cache-side state like the bf16 step.
    B, h, kp, b, r = 1024, 8, 8192, 128, 64
    deq = (codes.view(torch.float8_e4m3fn).float() * scales[..., None]).to(torch.bfloat16)
    pooled = api.pool_blocks(deq.view(torch.int16), B)
    reps = api.pool_blocks(deq.view(torch.int16), b)
    del deq
    ws_m = torch.empty(api.misa_route_ws(shape, B, h, kp, True), dtype=torch.uint8, device=dev)
    ws_h = torch.empty(api.hisa_coarse_fine_ws(shape, b, r, True), dtype=torch.uint8, device=dev)
    sel = {}
    for name, fn in (
            ("misa", lambda: api.misa_route_fp8(q, w, codes, scales, off, k, B, h, 0, pooled=pooled,
                                                want_heads=False, out_idx=oi, out_score=osc,
                                                ws=ws_m)),
            ("misa_dagger", lambda: api.misa_route_fp8(q, w, codes, scales, off, k, B, h, kp,
                                                       pooled=pooled, want_heads=False,
                                                       out_idx=oi, out_score=osc, ws=ws_m)),
            ("hisa", lambda: api.hisa_coarse_fine_fp8(q, w, codes, scales, off, k, b, r,
                                                      reps=reps, want_blocks=False, out_idx=oi,
                                                      out_score=osc, ws=ws_h))):
        ms_s, kern_s = flushed_calls(api, torch, fn, flush, steps)
        sel[name] = {"ms_per_call": ms_s, "kernels_us": {n: round(v, 2) for n, v in kern_s.items()}}
    return {"workload": "decode_128k_b8_h64_fp8keys", "cache": "cold: a 1 GiB read before "
            "each call", "ms_per_call": ms, "scores_per_s": Bt * L / (ms * 1e-3),
            "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in kern.items()},
            "roofline": {"kernel": "scan_dsa_fp8", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("scan_dsa_fp8", scan8_digest),
                         "algorithmic_bytes_per_launch": scan_bytes, "avg_us": round(us, 2)},
            "quantize": {"avg_us": round(q_us, 2), "algorithmic_bytes_per_launch": q_bytes,
                         "GB/s": round(q_bytes / (q_us * 1e-6) / 1e9, 1)},
            "fp8q": {"workload": "decode_128k_b8_h64_fp8keys_fp8q",
                     "what": "query converted to E4M3 in the kernel, 16x16x128 fp8 MFMA",
                     "ms_per_call": ms_q, "scores_per_s": Bt * L / (ms_q * 1e-3),
                     "kernels_us": {n: round(v, 2) for n, v in kern_q.items()},
                     "roofline": {"kernel": "scan_dsa_fp8q", "bound": "hbm",
                                  "achieved": round(gbs_q, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(gbs_q / HBM_PEAK_GBS, 4),
                                  "traffic": measured_traffic("scan_dsa_fp8q", scan8_digest),
                                  "algorithmic_bytes_per_launch": scan_bytes,
                                  "avg_us": round(us_q, 2)}},
            "selectors": {"config": {"B": B, "h": h, "k_prime": kp, "b": b, "r": r,
                                     "pools": "given: block means of the dequantized keys"},
                          **sel}}


def _flushed_ms(torch, call, flush, steps):
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        flush()
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps


def flushed_calls(api, torch, call, flush, steps):
    """Per-call time (events around each call, after a cache flush; the
    library's own kernel events off) and, from a second pass with them on,
    the library's per-kernel averages.  The flush kernel runs long enough for
    the host to enqueue the whole call behind it, so the call's host-side
    work is not in the time."""
    settle(call, torch, torch.device("cuda:0"))
    ms = _flushed_ms(torch, call, flush, steps)
    api.profile_enable(True)
    for _ in range(steps):
        flush()
        call()
    torch.cuda.synchronize()
    kern = api.profile_read()
    api.profile_enable(False)
    return ms, {n: 1e3 * tt / c for n, (tt, c) in kern.items()}


def flushed_graph_ms(torch, call, flush, steps):
    """Per-call time of the call captured alone into a HIP graph, replayed
    after a cache flush."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        flush()
        g.replay()
    torch.cuda.synchronize()
    return _flushed_ms(torch, g.replay, flush, steps)


def bench_lisa_resmisa(api, torch, dev, q, w, K, shape, flush, steps):
    """LISA (linear score g . k) and ResMiSA (block 128, r = 7 residual heads,
    extrema given as cache-side state) on the same decode batch."""
    Bt, L, H, d, off, k = shape.batch, shape.L, shape.H, shape.d, shape.causal_offset, shape.topk
    block, r = 128, 7
    oi = torch.empty((Bt, 1, k), dtype=torch.int32, device=dev)
    osc = torch.empty((Bt, 1, k), dtype=torch.float32, device=dev)
    ws_l = torch.empty(api.lisa_score_topk_ws(shape), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(api.resmisa_route_ws(shape, block, r, True), dtype=torch.uint8, device=dev)
    ext = api.block_extrema(K, block)
    heads = torch.empty((Bt, 1, r), dtype=torch.int32, device=dev)

    def lisa():
        api.lisa_score_topk(q, w, K, off, k, oi, osc, ws=ws_l)

    def resmisa():
        api.resmisa_route(q, w, K, off, k, block, r, extrema=ext, out_heads=heads, out_idx=oi,
                          out_score=osc, ws=ws_r)

    def ext_pass():
        api.block_extrema(K, block, out=ext)

    scan_nbytes = lambda hp: Bt * L * d * 2 + Bt * hp * d * 2 + Bt * hp * 4 + Bt * L * 4
    out = []
    for name, call, hp in (("lisa", lisa, 4), ("resmisa", resmisa, 4 + r)):
        ms, kus = flushed_calls(api, torch, call, flush, steps)
        nb = scan_nbytes(hp)
        gbs = nb / (kus["scan_dsa"] * 1e-6) / 1e9
        o = {"workload": "decode_128k_b8_h64_" + name, "cache": "cold: a 1 GiB read before each call",
             "ms_per_call": ms, "scores_per_s": Bt * L / (ms * 1e-3),
             "kernels_us": {n: round(v, 2) for n, v in kus.items()},
             "head_rows": hp,
             "roofline": {"kernel": "scan_dsa", "bound": "hbm", "achieved": round(gbs, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                          "algorithmic_bytes_per_launch": nb,
                          "avg_us": round(kus["scan_dsa"], 2)}}
        if name == "resmisa":
            o["config"] = {"block": block, "r": r, "extrema": "given (cache-side state)"}
            ems, ekus = flushed_calls(api, torch, ext_pass, flush, steps)
            eb = Bt * L * d * 2 + Bt * (L // block) * 2 * d * 2
            o["extrema_pass"] = {"avg_us": round(ekus["block_extrema"], 2),
                                 "algorithmic_bytes_per_launch": eb,
                                 "GB/s": round(eb / (ekus["block_extrema"] * 1e-6) / 1e9, 1)}
        out.append(o)
    return out[0], out[1]


def bench_misa_hisa(api, torch, dev, q, w, K, shape, reps_b, reps_B, flush, steps):
    """MISA x HISA on the same decode batch: h = 8 routed heads (B = 1024)
    score the b = 128 blocks, r = 64 blocks kept, every head rescores their
    8192 tokens; the pools are given (cache-side state, as in the step)."""
    Bt, k = shape.batch, shape.topk
    B, h, b, r = 1024, 8, 128, 64
    oi = torch.empty((Bt, 1, k), dtype=torch.int32, device=dev)
    osc = torch.empty((Bt, 1, k), dtype=torch.float32, device=dev)
    heads = torch.empty((Bt, 1, h), dtype=torch.int32, device=dev)
    blocks = torch.empty((Bt, 1, r), dtype=torch.int32, device=dev)
    ws = torch.empty(api.misa_hisa_ws(shape, B, h, b, r, True, True), dtype=torch.uint8,
                     device=dev)

    def call():
        api.misa_hisa(q, w, K, shape.causal_offset, k, B, h, b, r, pooled=reps_B, reps=reps_b,
                      out_heads=heads, out_blocks=blocks, out_idx=oi, out_score=osc, ws=ws)

    ms, kus = flushed_calls(api, torch, call, flush, steps)
    return {"workload": "decode_128k_b8_h64_misa_hisa", "cache": "cold: a 1 GiB read before "
            "each call", "config": {"B": B, "h": h, "b": b, "r": r, "pools": "given"},
            "ms_per_call": ms, "scores_per_s": Bt * shape.L / (ms * 1e-3),
            "kernels_us": {n: round(v, 2) for n, v in kus.items()}}


def bench_tidy_ragged(api, torch, dev, q, w, K, shape, outs, flush, steps):
    """The tidy-up of the DSA selector's 8 x 2048 indices (64-token pages), and
    the DSA selector on a ragged batch of the same capacity: lengths 128K,
    96K, 64K, 32K, 16K, 8K, 4K and 1K against the same batch padded to 128K."""
    Bt, L, k = shape.batch, shape.L, shape.topk
    idx = outs["dsa"][0]
    slots = torch.empty_like(idx)
    stats = torch.empty((Bt, 1, 3), dtype=torch.int32, device=dev)

    def tidy():
        api.tidy_indices(idx, 1, page_size=64, max_slots=L, out_slots=slots, out_stats=stats)

    ms_t, kus_t = flushed_calls(api, torch, tidy, flush, steps)
    st = stats.view(Bt, 3).cpu()
    tidy_o = {"workload": "decode_128k_b8_h64_tidy", "page_size": 64, "k": k, "max_slots": L,
              "avg_us": round(kus_t["tidy"], 2), "ms_per_call": ms_t,
              "mean_pages_per_row": float(st[:, 1].float().mean()),
              "mean_runs_per_row": float(st[:, 2].float().mean())}
    lens = [L, L * 3 // 4, L // 2, L // 4, L // 8, L // 16, L // 32, L // 128][:Bt]
    gl = torch.tensor(lens, dtype=torch.int32, device=dev)
    oi = torch.empty((Bt, 1, k), dtype=torch.int32, device=dev)
    osc = torch.empty((Bt, 1, k), dtype=torch.float32, device=dev)
    ws = torch.empty(api.indexer_score_topk_ragged_ws(shape), dtype=torch.uint8, device=dev)

    def ragged():
        api.indexer_score_topk_ragged(q, w, K, gl, k, total_len=sum(lens), out_idx=oi,
                                      out_score=osc, ws=ws)

    ms_r, kus_r = flushed_calls(api, torch, ragged, flush, steps)
    full = torch.full((Bt,), L, dtype=torch.int32, device=dev)

    def padded():
        api.indexer_score_topk_ragged(q, w, K, full, k, total_len=Bt * L, out_idx=oi,
                                      out_score=osc, ws=ws)

    ms_p, kus_p = flushed_calls(api, torch, padded, flush, steps)
    ragged_o = {"workload": "decode_b8_h64_ragged", "seq_lens": lens,
                "ms_per_call": ms_r, "scores_per_s": sum(lens) / (ms_r * 1e-3),
                "kernels_us": {n: round(v, 2) for n, v in kus_r.items()},
                "padded_ms_per_call": ms_p,
                "padded_kernels_us": {n: round(v, 2) for n, v in kus_p.items()}}
    return tidy_o, ragged_o


def bench_prefill(api, synth, torch, np, dev, iters):
    """Fused causal prefill: T = 4096 queries over 28672 cached keys, k = 2048."""
    p = synth.make_config("prefill_chunked")
    q = torch.from_numpy(p["q"].view(np.int16)).to(dev)
    w = torch.from_numpy(p["w"]).to(dev)
    K = torch.from_numpy(p["K"].view(np.int16)).to(dev)
    T, L, H, d, off, k = p["T"], p["L"], p["H"], p["d"], p["offset"], 2048
    shape = api.Shape(1, T, H, d, L, off, k)
    ws = torch.empty(api.indexer_score_topk_ws(shape), dtype=torch.uint8, device=dev)
    oi = torch.empty((1, T, k), dtype=torch.int32, device=dev)
    osc = torch.empty((1, T, k), dtype=torch.float32, device=dev)
    settle(lambda: api.indexer_score_topk(q, w, K, off, k, oi, osc, ws=ws), torch, dev)
    api.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(iters):
        api.indexer_score_topk(q, w, K, off, k, oi, osc, ws=ws)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    kern = api.profile_read()
    api.profile_enable(False)
    from sparse_attention_token_dsa_amd import workload as wl
    pairs = wl.legal_pairs(T, off)                      # legal (query, key) pairs
    flops = 2.0 * wl.indexer_macs(pairs, H, d)
    pf_us = 1e3 * kern["prefill_fused"][0] / kern["prefill_fused"][1]
    tflops = flops / (pf_us * 1e-6) / 1e12
    return {"workload": "prefill_chunked_T4096_P28672_h64", "ms_per_call": (t1 - t0) * 1e3 / iters,
            "logical_scores_per_s": pairs / ((t1 - t0) / iters),
            "topk_rows_per_s": T / ((t1 - t0) / iters),
            "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in kern.items()},
            "roofline": {"kernel": "prefill_fused", "bound": "mfma", "achieved": round(tflops, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(
                             "prefill_fused",
                             source_digest(["prefill.hip", "sa_frag.h", "sa_common.h"])),
                         "algorithmic_flops_per_launch": flops,
                         "counters": measured_mfma(
                             source_digest(["prefill.hip", "sa_frag.h", "sa_common.h"]))},
            "ragged": bench_prefill_ragged(api, synth, torch, np, dev, iters),
            "selectors": bench_prefill_selectors(api, torch, dev, q, w, K, shape, iters, pairs,
                                                 (t1 - t0) * 1e3 / iters),
            "fp8q": bench_prefill_fp8q(api, torch, dev, q, w, K, shape, oi, osc, iters, flops,
                                       pairs)}


def bench_prefill_selectors(api, torch, dev, q, w, K, shape, iters, pairs, dsa_ms):
    """MISA (h = 8 of 64 heads, B = 1024), MISA-dagger (k' = 8192) and HISA
    (b = 128, r = 64) on the same prefill chunk, block means given (cache-side
    state, pooled once outside the timing).  Prefill rows are where the
    indexer is MFMA-bound on this chip, so the head reduction shows here:
    MISA's rows go through the fused prefill on the routed heads' q rows."""
    T, off, k = shape.T, shape.causal_offset, shape.topk
    H, d, L = shape.H, shape.d, shape.L
    B, h, kp, b, r = 1024, 8, 8192, 128, 64
    pooled = api.pool_blocks(K, B)
    reps = api.pool_blocks(K, b)
    oi = torch.empty((1, T, k), dtype=torch.int32, device=dev)
    osc = torch.empty((1, T, k), dtype=torch.float32, device=dev)
    ws_m = torch.empty(api.misa_route_ws(shape, B, h, 0, True), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(api.misa_route_ws(shape, B, h, kp, True), dtype=torch.uint8, device=dev)
    ws_h = torch.empty(api.hisa_coarse_fine_ws(shape, b, r, True), dtype=torch.uint8,
                       device=dev)
    calls = {
        "misa": lambda: api.misa_route(q, w, K, off, k, B, h, 0, pooled=pooled,
                                       want_heads=False, out_idx=oi, out_score=osc, ws=ws_m),
        "misa_dagger": lambda: api.misa_route(q, w, K, off, k, B, h, kp, pooled=pooled,
                                              want_heads=False, out_idx=oi, out_score=osc,
                                              ws=ws_d),
        "hisa": lambda: api.hisa_coarse_fine(q, w, K, off, k, b, r, reps=reps,
                                             want_blocks=False, out_idx=oi, out_score=osc,
                                             ws=ws_h),
    }
    out = {"workload": "prefill_chunked_T4096_P28672_h64",
           "config": {"B": B, "h": h, "k_prime": kp, "b": b, "r": r,
                      "pools": "given (block means of the cached keys)"},
           "dsa_ms_per_call": dsa_ms}
    for name, call in calls.items():
        settle(call, torch, dev)
        api.profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(iters):
            call()
        torch.cuda.synchronize(dev)
        t1 = time.perf_counter()
        kern = api.profile_read()
        api.profile_enable(False)
        ms = (t1 - t0) * 1e3 / iters
        out[name] = {"ms_per_call": ms, "dsa_over_this": dsa_ms / ms,
                     "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in kern.items()}}
    # the routed prefill's own contraction: h heads per legal pair
    from sparse_attention_token_dsa_amd import workload as wl
    flops = 2.0 * wl.misa_macs(pairs, h, d)
    us = out["misa"]["kernels_us"].get("prefill_fused")
    if us:
        tf = flops / (us * 1e-6) / 1e12
        out["misa"]["routed_prefill"] = {
            "kernel": "prefill_fused", "algorithmic_flops_per_launch": flops,
            "achieved_tflops": round(tf, 1), "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "note": "8 routed heads fill half of the kernel's one 16-row head tile, and the "
                    "per-pair epilogue, threshold and survivor work does not shrink with the "
                    "head count"}
    return out


def bench_prefill_fp8q(api, torch, dev, q, w, K, shape, oi, osc, iters, flops, pairs):
    """The same chunked prefill on the FP8 key cache with the query converted
    to E4M3 in the kernel (indexer_score_topk_fp8q): the contraction on the
    16x16x128 fp8 MFMA, against the dense fp8 peak."""
    T, off, k = shape.T, shape.causal_offset, shape.topk
    digest = source_digest(["prefill.hip", "sa_frag.h", "sa_common.h"])
    codes, scales = api.quantize_keys_fp8(K)
    ws = torch.empty(api.indexer_score_topk_fp8q_ws(shape), dtype=torch.uint8, device=dev)

    def call():
        api.indexer_score_topk_fp8q(q, w, codes, scales, off, k, oi, osc, ws=ws)
    settle(call, torch, dev)
    api.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(iters):
        call()
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    kern = api.profile_read()
    api.profile_enable(False)
    us = 1e3 * kern["prefill_fused_fp8q"][0] / kern["prefill_fused_fp8q"][1]
    tflops = flops / (us * 1e-6) / 1e12
    return {"workload": "prefill_chunked_T4096_P28672_h64_fp8keys_fp8q",
            "what": "keys as E4M3 codes + one fp32 scale per key, query quantized per head "
                    "in the kernel, 16x16x128 fp8 MFMA",
            "ms_per_call": (t1 - t0) * 1e3 / iters,
            "logical_scores_per_s": pairs / ((t1 - t0) / iters),
            "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in kern.items()},
            "roofline": {"kernel": "prefill_fused_fp8q", "bound": "mfma",
                         "achieved": round(tflops, 1), "peak": FP8_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / FP8_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_fused_fp8q", digest),
                         "algorithmic_flops_per_launch": flops,
                         "vs_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "counters": measured_mfma(digest, "prefill_fused_fp8q_mfma")}}


def bench_prefill_ragged(api, synth, torch, np, dev, iters):
    """Chunked prefill of sequences with different cached prefixes: 4 sequences
    of 1024 new queries each at lengths 32K, 24K, 12K and 4K (capacity 32K),
    one ragged call, next to the same batch padded to the capacity."""
    Bt, T, L, H, d, k = 4, 1024, 32768, 64, 128, 2048
    lens = [32768, 24576, 12288, 4096]
    p = synth.make_problem(611, Bt=Bt, T=T, L=L, H=H, d=d, offset=L - T, needles=16,
                           needle_mode="rows")
    q = torch.from_numpy(p["q"].view(np.int16)).to(dev)
    w = torch.from_numpy(p["w"]).to(dev)
    K = torch.from_numpy(p["K"].view(np.int16)).to(dev)
    gl = torch.tensor(lens, dtype=torch.int32, device=dev)
    full = torch.full((Bt,), L, dtype=torch.int32, device=dev)
    shape = api.Shape(Bt, T, H, d, L, L - T, k)
    ws = torch.empty(api.indexer_score_topk_ragged_ws(shape), dtype=torch.uint8, device=dev)
    oi = torch.empty((Bt, T, k), dtype=torch.int32, device=dev)
    osc = torch.empty((Bt, T, k), dtype=torch.float32, device=dev)
    res = {}
    for name, sl, ls in (("ragged", gl, lens), ("padded", full, [L] * Bt)):
        def call(sl=sl):
            api.indexer_score_topk_ragged(q, w, K, sl, k, out_idx=oi, out_score=osc, ws=ws)
        settle(call, torch, dev)
        api.profile_enable(True)
        for _ in range(iters):
            call()
        torch.cuda.synchronize(dev)
        kern = api.profile_read()
        api.profile_enable(False)
        us = 1e3 * kern["prefill_fused"][0] / kern["prefill_fused"][1]
        pairs = sum(n - T + i + 1 for n in ls for i in range(T))
        res[name] = {"prefill_us": round(us, 1), "legal_pairs": pairs,
                     "TFLOP/s": round(2.0 * pairs * H * d / (us * 1e-6) / 1e12, 1)}
    return {"workload": "prefill_ragged_b4_T1024_cap32k_h64", "seq_lens": lens, "T": T,
            "k": k, **res}


def host_cpu():
    """CPU model, logical CPUs of the host and the CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    return model, os.cpu_count() or 1, usable


def cpu_baseline(p, k, B, h, kp, b, r, gpu_sets):
    """The fp64 CPU oracle on all 8 query rows of the same workload, through the
    same four selectors (pooling included in its MISA / HISA calls), one
    thread per row.  It selects k + 1 per row, so the same run also gives the
    cutoff margin S_k - S_(k+1) of each row and selector, and how many of the
    oracle's top-k the GPU exchanged for near-tie positions."""
    import numpy as np

    import oracle
    model, ncpu, usable = host_cpu()
    rows = p["Bt"] * p["T"]
    threads = min(usable, rows)
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    t0 = time.perf_counter()
    res = {"dsa": oracle.dsa(prob, k + 1, nthreads=threads),
           "misa": oracle.misa(prob, k + 1, B, h, 0, nthreads=threads),
           "misa_dagger": oracle.misa(prob, k + 1, B, h, kp, nthreads=threads),
           "hisa": oracle.hisa(prob, k + 1, b, r, nthreads=threads)}
    dt = time.perf_counter() - t0
    pairs = 4 * rows * p["L"]
    base = {"value": pairs / dt, "unit": "scores/s", "cores": threads, "kind": "oracle",
            "host_cpu_model": model, "host_logical_cpus": ncpu, "usable_cpus": usable,
            "sample": "all %d query rows of the L=%d decode batch through DSA, MISA, "
                      "MISA-dagger and HISA (fp64 C oracle, %d threads, one per row); "
                      "%.1f s wall" % (rows, p["L"], threads, dt)}
    margins = {}
    for m, o in res.items():
        idx, sc = (o[0], o[1]) if isinstance(o, tuple) else (o["idx"], o["score"])
        rel, diff = [], []
        for row in range(rows):
            s_k, s_k1 = sc[row, k - 1], sc[row, k]
            top = float(np.max(np.abs(sc[row][np.isfinite(sc[row])])))
            rel.append((s_k - s_k1) / top if np.isfinite(s_k1) and top > 0 else float("inf"))
            diff.append(len(set(idx[row, :k].tolist()) - set(gpu_sets[m][row].tolist())))
        margins[m] = {"min_rel_margin": float(np.min(rel)),
                      "median_rel_margin": float(np.median(rel)),
                      "rows_margin_below_tol": int(np.sum(np.array(rel) < 2e-3)),
                      "exchanged_positions": int(np.sum(diff)),
                      "rows_with_exchanges": int(np.sum(np.array(diff) > 0))}
    return base, {"what": "oracle cutoff margin (S_k - S_(k+1)) / max|S| per row, and oracle "
                          "top-k positions the GPU set replaced (near ties; the parity tests "
                          "bound them), 8 rows per selector",
                  **margins}


if __name__ == "__main__":
    main()
