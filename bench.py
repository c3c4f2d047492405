#!/usr/bin/env python3
"""Benchmark of the CSA hot path on one MI355X (gfx950).

Headline: decode queries/s on a batch of 8 sequences with 131072-token
contexts (m = 4 -> 32768 compressed entries each, c = 512, c^I = 128,
64 indexer heads, 64 attention heads, top-1024).  One step = the whole decode
path for one batch: the lightning-indexer sweep over every compressed key,
the top-k selection, and the shared-KV sparse MQA with its split merge.

Inputs are seeded synthetic tensors, resident in HBM before timing starts.
A decode step streams ~73 MiB, which would otherwise sit in the 256 MB
Infinity Cache between steps; the timed steps therefore rotate through
--replicas device copies of the inputs (8 by default: > 512 MiB of key
sweeps), the way a server alternates between batches.  The warm-cache rate
(one copy) is reported beside it.

Also reported on the same line: the per-kernel durations measured with HIP
events recorded on the launch stream around every library kernel of the
timed steps (a second pass over the same steps), the roofline of the
dominant kernel, the prefill of one 32768-token sequence (tokens/s), and the
CPU oracle on a bounded sample of the decode workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def _kernel_stats(api, names):
    out = {}
    for n in names:
        ms, cnt = api.csa_timing_read(n)
        if cnt:
            out[n] = {"launches": cnt, "avg_us": 1000.0 * ms / cnt, "total_ms": ms}
    return out


def _traffic(kernel: str, key: str = "hbm_bytes_per_launch"):
    """HBM bytes per launch (or the record's `key`) from committed counter runs, while the kernel's sources are
    unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for src in rec.get("sources", []):
        with open(os.path.join(ROOT, "compressed_sparse_attention_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    if rec.get("sources_sha256") != h.hexdigest():
        return None
    return rec.get(key)


def per_step_stats(torch, run_one, n_pool, steps):
    """Per-step durations (us) of `steps` back-to-back steps, from an event recorded on the launch stream
    after every step: median and 10th / 90th percentiles."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        run_one(i % n_pool)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(steps)])
    return {"n": steps, "median_us": round(float(np.median(t)), 3), "p10_us": round(float(np.percentile(t, 10)), 3),
            "p90_us": round(float(np.percentile(t, 90)), 3), "mean_us": round(float(t.mean()), 3)}


def bench_decode(args, torch, api, synth, layer):
    w = synth.WORKLOADS[4]
    dev = "cuda:0"
    D = synth.make_decode(w)
    B = int(D["seq_len"].shape[0])
    max_cand = int(D["n_blocks"].max())
    base = {
        "q": layer.to_device(D["q"], w.dtype, dev),
        "qI": layer.to_device(D["qI"], w.dtype, dev),
        "wI": layer.to_device(D["wI"], "f32", dev),
        "C": layer.to_device(D["Ccomp"], w.dtype, dev),
        "K": layer.to_device(D["KIcomp"], w.dtype, dev),
    }
    reps = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(args.replicas - 1)]
    seq_len = torch.from_numpy(D["seq_len"]).to(dev)
    off = torch.from_numpy(D["kv_offset"]).to(dev)
    buf = layer.DecodeBuffers(B, w.k, w.nh, w.c, w.nhI, max_cand, base["q"].dtype, dev)

    def step(i, pool):
        r = pool[i % len(pool)]
        layer.decode(r["q"], r["qI"], r["wI"], r["C"], r["K"], seq_len, off, w.m, w.k, max_cand, buf=buf)

    def timed(run_one, n_pool, steps, warmup):
        for i in range(warmup):
            run_one(i % n_pool)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            run_one(i % n_pool)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # eager reference output of copy 0, then one HIP graph per input copy
    step(0, reps)
    torch.cuda.synchronize()
    ref_idx, ref_o = buf.idx.clone(), buf.o.clone()
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0, reps)
    torch.cuda.current_stream().wait_stream(side)
    for i in range(len(reps)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i, reps)
        graphs.append(g)
    for _ in range(3):  # replays, with eager work in between, must reproduce the eager result
        buf.idx.fill_(-7)
        graphs[0].replay()
        torch.cuda.synchronize()
        if not (torch.equal(buf.idx, ref_idx) and torch.equal(buf.o, ref_o)):
            raise RuntimeError("graph replay differs from the eager decode step")
        step(1, reps)
        torch.cuda.synchronize()

    ms_eager = timed(lambda i: step(i, reps), len(reps), args.steps, args.warmup)
    ms = timed(lambda i: graphs[i].replay(), len(reps), args.steps, args.warmup)
    print(f"[bench] decode: {ms * 1000:.2f} us/step over {args.steps} graph replays "
          f"({len(reps)} input copies); eager launches {ms_eager * 1000:.2f} us/step", flush=True)
    ms_warm = timed(lambda i: graphs[0].replay(), 1, args.steps, args.warmup)
    print(f"[bench] decode warm cache: {ms_warm * 1000:.2f} us/step", flush=True)
    n_dist = max(100, args.steps)
    dist = {"eager": per_step_stats(torch, lambda i: step(i, reps), len(reps), n_dist),
            "graph": per_step_stats(torch, lambda i: graphs[i].replay(), len(reps), n_dist)}
    for k_, d_ in dist.items():
        print(f"[bench] decode {k_} per step over {d_['n']} steps: median {d_['median_us']:.2f} us, "
              f"p10 {d_['p10_us']:.2f}, p90 {d_['p90_us']:.2f}", flush=True)

    # second pass over the same steps with per-kernel HIP events on the launch stream
    api.csa_timing_reset()
    api.csa_timing_enable(True)
    timed(lambda i: step(i, reps), len(reps), args.steps, 0)
    api.csa_timing_enable(False)
    kern = _kernel_stats(api, ["hist_clear", "indexer_sweep", "topk", "mqa", "mqa_combine"])
    api.csa_timing_reset()
    for n, s in kern.items():
        print(f"[bench]   {n:14s} {s['avg_us']:8.2f} us/launch", flush=True)

    # algorithmic bytes of the indexer sweep per query: every candidate key of the
    # sequence (N_b * cI bf16), the query's indexer heads and head weights
    N = max_cand
    sweep_bytes = B * (2 * N * w.cI + 2 * w.nhI * w.cI + 4 * w.nhI)
    # whole decode step per query: key sweep + gathered entries + q + o + selected indices
    step_bytes = B * (2 * N * w.cI + 2 * min(w.k, N) * w.c + 2 * (w.nh * w.c + w.nhI * w.cI) + 4 * w.nhI
                      + 2 * w.nh * w.c + 4 * w.k)
    name = "indexer_sweep"
    sw = kern.get(name)
    roof = None
    if sw:
        achieved = sweep_bytes / (sw["avg_us"] * 1e-6) / 1e9
        roof = {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": _traffic(name),
                "algorithmic_bytes_per_launch": sweep_bytes}
    return {
        "workload": w, "B": B, "ms": ms, "ms_warm": ms_warm, "ms_eager": ms_eager, "kernels": kern, "roofline": roof,
        "dist": dist,
        "step_bytes": step_bytes, "max_cand": max_cand, "D": D,
    }


def bench_prefill(args, torch, api, synth, layer, selection="dense", HW=None):
    """The 32768-token prefill; selection "dense" (score matrix, then selector) or "stream" (the indexer
    keeps only selectable scores).  HW: (H, W) already on the device, or None."""
    w = synth.WORKLOADS[3]
    dev = "cuda:0"
    if HW is None:
        P = synth.make_prefill(w)
        HW = (layer.to_device(P["H"], w.dtype, dev), layer.pack_prefill_params(P, w.dtype, dev))
        del P
    H, W = HW
    buf = layer.PrefillBuffers(w.n, w.m, w.k, w.nh, w.nhI, w.c, w.cI, w.dc, H.dtype, dev, selection=selection)

    def run(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            layer.prefill(H, W, w.m, w.k, w.nh, w.nhI, buf=buf)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    run(max(1, args.prefill_warmup))
    ms = run(args.prefill_steps)
    api.csa_timing_reset()
    api.csa_timing_enable(True)
    run(args.prefill_steps)
    api.csa_timing_enable(False)
    kern = _kernel_stats(api, ["gemm", "compress", "indexer_prefill", "topk", "mqa", "mqa_combine"])
    api.csa_timing_reset()
    print(f"[bench] prefill ({selection} selection): {ms:.2f} ms per {w.n}-token sequence", flush=True)
    for n, s in kern.items():
        print(f"[bench]   {n:16s} {s['total_ms'] / args.prefill_steps:9.3f} ms/step "
              f"({s['launches'] // args.prefill_steps} launches)", flush=True)
    n_pairs = sum(t // w.m for t in range(w.n))
    idx_flops = 2.0 * n_pairs * w.nhI * w.cI
    ip = kern.get("indexer_prefill")
    roof = None
    if ip:
        ach = idx_flops / (ip["avg_us"] * 1e-6) / 1e12
        roof = {"kernel": "indexer_prefill", "bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                "traffic": _traffic("indexer_prefill") if selection == "dense" else None,
                "algorithmic_flops_per_launch": idx_flops}
    out = {"workload": w.name, "selection": selection, "tokens": w.n, "ms": ms, "tokens_per_s": w.n / (ms * 1e-3),
           "kernels_ms_per_step": {n: round(s["total_ms"] / args.prefill_steps, 4) for n, s in kern.items()},
           "indexer_roofline": roof, "stage_rooflines": _prefill_stage_rooflines(w, kern, args.prefill_steps)}
    del buf
    return out, HW


def bench_selection_long(args, torch, api, synth, layer):
    """Eqs 8-9 alone on one longer sequence, materialised against streaming selection: 65536 query tokens,
    16384 compressed blocks (m = 4), the 32768-token layer's indexer widths (64 heads of 128) and k = 512.
    Inputs are drawn on the GPU from a seeded generator (queries std 128^-1/2, keys and head weights N(0, 1));
    the two paths' selections are compared as sets on every row (they must agree except within the top-k
    comparison band, which on these continuous scores means equality)."""
    dev = "cuda:0"
    n, m, nhI, cI, k = 65536, 4, 64, 128, 512
    N = n // m
    g = torch.Generator(device=dev)
    g.manual_seed(51)
    qI = (torch.randn(n, nhI, cI, generator=g, device=dev) / math.sqrt(cI)).to(torch.bfloat16)
    K = torch.randn(N, cI, generator=g, device=dev).to(torch.bfloat16)
    wI = torch.randn(n, nhI, generator=g, device=dev)
    out = {}
    idx = {}
    for sel in ("dense", "stream"):
        ix = torch.empty(n, k, dtype=torch.int32, device=dev)
        if sel == "dense":
            ws = torch.empty(api.csa_index_topk_workspace(n, N, nhI, k), dtype=torch.uint8, device=dev)
            fn = lambda: api.csa_index_topk(qI, wI, K, m, k, N, ix, workspace=ws)  # noqa: E731
        else:
            ws = torch.empty(api.csa_index_topk_stream_workspace(n, N), dtype=torch.uint8, device=dev)
            fn = lambda: api.csa_index_topk_stream(qI, wI, K, m, k, N, ix, workspace=ws)  # noqa: E731
        fn()
        torch.cuda.synchronize()
        api.csa_timing_reset()
        api.csa_timing_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.prefill_steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        api.csa_timing_enable(False)
        kern = _kernel_stats(api, ["indexer_prefill", "topk"])
        api.csa_timing_reset()
        ms = e0.elapsed_time(e1) / args.prefill_steps
        out[sel] = {"ms": round(ms, 4), "kernels_ms": {kk: round(v["total_ms"] / args.prefill_steps, 4)
                                                       for kk, v in kern.items()}}
        print(f"[bench] selection of {n} tokens x {N} blocks, {sel}: {ms:.3f} ms "
              f"{out[sel]['kernels_ms']}", flush=True)
        idx[sel] = ix
        del ws
    a = torch.sort(idx["dense"], dim=1).values
    b = torch.sort(idx["stream"], dim=1).values
    out["rows_with_equal_sets"] = int((a == b).all(dim=1).sum())
    out["workload"] = f"selection_n{n}_N{N}_k{k}_bf16"
    return out


def _prefill_stage_rooflines(w, kern, steps):
    """Algorithmic work of the other prefill stages per pass against their bound: the projections (eqs 1, 2, 5,
    6, 7, 10) and the attention (eq 11) on bf16 MFMA; compression (eqs 3-4, main and indexer) and the top-k
    (eq 9: reading each token's causal scores, writing its k indices) on HBM."""
    n, d, m, k = w.n, w.d, w.m, w.k
    width = 4 * w.c + 4 * w.cI + w.dc
    ncand = [t // m for t in range(n)]
    work = {
        "projections": ("gemm", "mfma", 2.0 * n * (d * width + d * w.nhI + w.dc * w.nhI * w.cI + w.dc * w.nh * w.c)),
        "compression": ("compress", "hbm", 2.0 * (4 * n * (w.c + w.cI) + (n // m) * (w.c + w.cI))),
        "topk": ("topk", "hbm", 4.0 * sum(ncand) + 4.0 * n * k),
        "mqa": ("mqa", "mfma", 4.0 * sum(min(k, x) for x in ncand) * w.nh * w.c),
    }
    out = {}
    for stage, (fam, bound, amount) in work.items():
        st = kern.get(fam)
        if not st:
            continue
        sec = st["total_ms"] / steps * 1e-3
        if bound == "mfma":
            ach, peak, unit, key = amount / sec / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "algorithmic_flops_per_step"
        else:
            ach, peak, unit, key = amount / sec / 1e9, HBM_PEAK_GBS, "GB/s", "algorithmic_bytes_per_step"
        out[stage] = {"kernels": fam, "bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit,
                      "frac": round(ach / peak, 4), key: amount}
    return out


def bench_other_configs(args, torch, api, synth, layer):
    """The other seeded workloads, timed on their own: the 512-token fp32 prefill (a parity-sized case, launch
    bound), the 32 x 8K decode batch and the ragged 64-sequence decode batch (m = 8, 128 heads).  Decode steps are
    eager launches over enough input copies to exceed the 256 MB last-level cache; their HBM fraction is the
    step's algorithmic bytes (every candidate key, the selected entries, queries, outputs and indices) over the
    step time against 8 TB/s."""
    dev = "cuda:0"
    out = {}

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    w = synth.WORKLOADS[1]
    P = synth.make_prefill(w)
    W = layer.pack_prefill_params(P, w.dtype, dev)
    H = layer.to_device(P["H"], w.dtype, dev)
    buf = layer.PrefillBuffers(w.n, w.m, w.k, w.nh, w.nhI, w.c, w.cI, w.dc, H.dtype, dev)
    ms = timed(lambda i: layer.prefill(H, W, w.m, w.k, w.nh, w.nhI, buf=buf), 50, 5)
    out[w.name] = {"kind": "prefill", "tokens": w.n, "ms": round(ms, 4), "tokens_per_s": round(w.n / (ms * 1e-3), 1)}
    print(f"[bench] {w.name}: {ms * 1000:.1f} us per {w.n}-token prefill", flush=True)

    for cfg in (2, 5):
        w = synth.WORKLOADS[cfg]
        D = synth.make_decode(w)
        B = int(D["seq_len"].shape[0])
        nb = D["n_blocks"].astype(np.int64)
        max_cand = int(nb.max())
        base = {"q": layer.to_device(D["q"], w.dtype, dev), "qI": layer.to_device(D["qI"], w.dtype, dev),
                "wI": layer.to_device(D["wI"], "f32", dev), "C": layer.to_device(D["Ccomp"], w.dtype, dev),
                "K": layer.to_device(D["KIcomp"], w.dtype, dev)}
        per_copy = sum(t.numel() * t.element_size() for t in base.values())
        copies = max(1, min(8, -(-(320 << 20) // per_copy)))
        reps = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
        seq_len = torch.from_numpy(D["seq_len"]).to(dev)
        off = torch.from_numpy(D["kv_offset"]).to(dev)
        dbuf = layer.DecodeBuffers(B, w.k, w.nh, w.c, w.nhI, max_cand, base["q"].dtype, dev)

        def step(i):
            r = reps[i % len(reps)]
            layer.decode(r["q"], r["qI"], r["wI"], r["C"], r["K"], seq_len, off, w.m, w.k, max_cand, buf=dbuf)

        ms = timed(step, 100, 10)
        api.csa_timing_reset()
        api.csa_timing_enable(True)
        timed(step, 50, 0)
        api.csa_timing_enable(False)
        kern = _kernel_stats(api, ["hist_clear", "indexer_sweep", "topk", "mqa", "mqa_combine"])
        api.csa_timing_reset()
        sel = np.minimum(nb, w.k)
        step_bytes = int((2 * nb * w.cI + 2 * sel * w.c + 2 * (w.nh * w.c + w.nhI * w.cI) + 4 * w.nhI
                          + 2 * w.nh * w.c + 4 * w.k).sum())
        gbs = step_bytes / (ms * 1e-3) / 1e9
        out[w.name] = {"kind": "decode", "batch": B, "us_per_step": round(ms * 1000, 3),
                       "queries_per_s": round(B / (ms * 1e-3), 1), "step_bytes": step_bytes,
                       "step_hbm_fraction": round(gbs / HBM_PEAK_GBS, 4), "input_copies": copies,
                       "kernels_us": {n: round(st["avg_us"], 3) for n, st in kern.items()}}
        print(f"[bench] {w.name}: {ms * 1000:.2f} us/step, {B / (ms * 1e-3):.0f} queries/s, "
              f"{gbs:.0f} GB/s of step bytes", flush=True)
        del reps, base, dbuf
    return out


def bench_prefill_backward(args, torch, api, synth, layer):
    """Backward of the 32768-token prefill (training): sparse-MQA gradients (dq and the key-gradient shares,
    grouped and summed per compressed entry), compression gradients, and the eq 10 and eqs 1, 2, 5 projection
    gradients (dX and dW), given a seeded random dL/do."""
    w = synth.WORKLOADS[3]
    dev = "cuda:0"
    P = synth.make_prefill(w)
    W = layer.pack_prefill_params(P, w.dtype, dev)
    H = layer.to_device(P["H"], w.dtype, dev)
    del P
    buf = layer.prefill(H, W, w.m, w.k, w.nh, w.nhI)
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    dO = torch.randn(w.n, w.nh, w.c, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    grads = layer.PrefillGrads(w.n, w.m, w.k, w.nh, w.c, w.cI, w.dc, w.d, H.dtype, dev)

    def run(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            layer.prefill_backward(H, W, buf, dO, w.m, w.k, w.nh, grads=grads)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    run(max(1, args.prefill_warmup))
    ms = run(args.prefill_steps)
    api.csa_timing_reset()
    api.csa_timing_enable(True)
    run(args.prefill_steps)
    api.csa_timing_enable(False)
    names = ["mqa_bwd", "mqa_bwd_zero", "mqa_bwd_sort", "mqa_bwd_reduce", "compress_bwd", "compress_bias_reduce",
             "transpose", "gemm"]
    kern = _kernel_stats(api, names)
    api.csa_timing_reset()
    print(f"[bench] prefill backward: {ms:.2f} ms per {w.n}-token sequence", flush=True)
    for n, st in kern.items():
        print(f"[bench]   {n:20s} {st['total_ms'] / args.prefill_steps:9.3f} ms/step "
              f"({st['launches'] // args.prefill_steps} launches)", flush=True)
    pairs = sum(min(w.k, t // w.m) for t in range(w.n))
    flops = 10.0 * w.nh * w.c * pairs  # S, dP, dq (nh c MACs each) and the two key-gradient paths (2 nh c)
    mb = kern.get("mqa_bwd")
    roof = None
    if mb:
        per_launch = mb["total_ms"] / mb["launches"]
        launches_per_step = mb["launches"] // args.prefill_steps
        ach = flops / launches_per_step / (per_launch * 1e-3) / 1e12
        roof = {"kernel": "mqa_bwd", "bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                "algorithmic_flops_per_step": flops, "launches_per_step": launches_per_step}
    return {"workload": w.name + "_backward", "tokens": w.n, "ms": round(ms, 4),
            "tokens_per_s": round(w.n / (ms * 1e-3), 1),
            "kernels_ms_per_step": {n: round(st["total_ms"] / args.prefill_steps, 4) for n, st in kern.items()},
            "mqa_bwd_roofline": roof}


def bench_prefill_varlen(args, torch, api, synth, layer):
    """Prefill of 16 packed sequences with ragged lengths (512 .. 4096 tokens, seeded draw) at the layer
    sizes of the 32768-token prefill: one call per stage for the whole batch, each sequence causal on its
    own."""
    w = synth.WORKLOADS[3]
    dev = "cuda:0"
    lengths = [int(x) for x in synth.ragged_lengths(synth.rng_for(41), 16, 512, 4096)]
    n = sum(lengths)
    P = synth.make_prefill(w, seed=42, n=n)
    W = layer.pack_prefill_params(P, w.dtype, dev)
    H = layer.to_device(P["H"], w.dtype, dev)
    del P
    buf = layer.VarlenPrefill(lengths, w.m, w.k, w.nh, w.nhI, w.c, w.cI, w.dc, H.dtype, dev)

    def run(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            layer.prefill_varlen(H, lengths, W, w.m, w.k, w.nh, w.nhI, buf=buf)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    run(max(1, args.prefill_warmup))
    ms = run(args.prefill_steps)
    api.csa_timing_reset()
    api.csa_timing_enable(True)
    run(args.prefill_steps)
    api.csa_timing_enable(False)
    kern = _kernel_stats(api, ["gemm", "compress", "varlen_meta", "indexer_prefill", "topk", "mqa", "mqa_combine"])
    api.csa_timing_reset()
    print(f"[bench] packed prefill: {ms:.2f} ms for {len(lengths)} sequences, {n} tokens", flush=True)
    pairs = sum(t // w.m for L in lengths for t in range(L))
    idx_flops = 2.0 * pairs * w.nhI * w.cI
    ip = kern.get("indexer_prefill")
    roof = None
    if ip:
        ach = idx_flops / (ip["avg_us"] * 1e-6) / 1e12
        roof = {"kernel": "indexer_prefill", "bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4), "algorithmic_flops_per_launch": idx_flops}
    return {"workload": "prefill_varlen_16seq_512-4096_bf16", "sequences": len(lengths), "tokens": n,
            "lengths": lengths, "ms": round(ms, 4), "tokens_per_s": round(n / (ms * 1e-3), 1),
            "kernels_ms_per_step": {k: round(v["total_ms"] / args.prefill_steps, 4) for k, v in kern.items()},
            "indexer_roofline": roof}


def bench_decode_step(args, torch, api, synth, layer):
    """Decode with cache maintenance: the batch of 8 sequences at 131072 tokens appends one token each.

    Layer sizes of the 32768-token prefill (d = 4096, d_c = 1536) with the decode batch's attention
    sizes; the caches hold seeded synthetic entries (the state a 131072-token prefill hands over),
    the rings random projected rows.  One step: four few-row projections (the weights are streamed
    once), two compress-and-appends, indexer sweep, top-k and sparse MQA; positions advance, so a
    block is appended every m steps.  Two copies of weights and state alternate (> 256 MB)."""
    import numpy as np
    wd, wp = synth.WORKLOADS[4], synth.WORKLOADS[3]
    dev = "cuda:0"
    B, L, m = wd.B, wd.L, wd.m
    N = L // m
    n_tok = 64  # pool of new hidden states per sequence
    P = synth.make_prefill(wp, seed=31, n=B * n_tok)
    Hpool = layer.to_device(P["H"], wp.dtype, dev).view(n_tok, B, wp.d)
    del P["H"]
    D = synth.make_decode(wd, seed=32)
    total = 3 * (args.steps + args.warmup) + 16
    cap = N + total // m + 8
    dt = torch.bfloat16
    rng = synth.rng_for(33)
    ring = layer.to_device(synth.normal(rng, (B, 2 * m, 4 * wd.c), 1.0, "bf16"), "bf16", dev)
    ring_I = layer.to_device(synth.normal(rng, (B, 2 * m, 4 * wd.cI), 1.0, "bf16"), "bf16", dev)
    C = layer.to_device(D["Ccomp"], wd.dtype, dev).view(B, N, wd.c)
    K = layer.to_device(D["KIcomp"], wd.dtype, dev).view(B, N, wd.cI)
    del D
    copies = []
    for r in range(2):
        W = layer.pack_prefill_params(P, wp.dtype, dev)
        st = layer.DecodeState(B, cap, m, wd.c, wd.cI, dt, dev)
        st.Ccomp.view(B, cap, wd.c)[:, :N].copy_(C)
        st.KIcomp.view(B, cap, wd.cI)[:, :N].copy_(K)
        st.ring.copy_(ring)
        st.ring_I.copy_(ring_I)
        st.t.fill_(L)
        st.t_host[:] = L
        bufr = layer.DecodeBuffers(B, wd.k, wd.nh, wd.c, wd.nhI, cap, dt, dev)
        copies.append((W, st, bufr))
    del C, K, P

    def step(i):
        W, st, bufr = copies[i % 2]
        layer.decode_step(Hpool[(i // 2) % n_tok], W, st, m, wd.k, wd.nh, wd.nhI, buf=bufr)

    def run(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    run(max(1, args.warmup))
    ms = run(args.steps)
    api.csa_timing_reset()
    api.csa_timing_enable(True)
    run(args.steps)
    api.csa_timing_enable(False)
    names = ["gemm_smallm", "compress_append", "hist_clear", "indexer_sweep", "topk", "mqa", "mqa_combine"]
    kern = _kernel_stats(api, names)
    api.csa_timing_reset()
    t_end = [int(c[1].t.max()) for c in copies]
    if max(t_end) > cap * m:
        raise RuntimeError("decode-step benchmark outgrew its cache capacity")
    print(f"[bench] decode step with cache maintenance: {ms * 1000:.2f} us/step (eager)", flush=True)
    for n, s_ in kern.items():
        print(f"[bench]   {n:16s} {s_['total_ms'] / args.steps * 1000:8.2f} us/step "
              f"({s_['launches'] // args.steps} launches)", flush=True)
    # weights streamed by the four projections of one step (bf16, two paired launches), plus their inputs and outputs
    d, dc, c, cI = wp.d, wp.dc, wd.c, wd.cI
    shapes = [(4 * c + 4 * cI + dc, d, 2), (wd.nhI, d, 4), (wd.nhI * cI, dc, 2), (wd.nh * c, dc, 2)]
    gemm_bytes = sum(n * k * 2 + B * k * 2 + B * n * ob for n, k, ob in shapes)
    g = kern.get("gemm_smallm")
    roof = None
    if g:
        t_step = g["total_ms"] / args.steps * 1e-3
        ach = gemm_bytes / t_step / 1e9
        roof = {"kernel": "gemm_smallm", "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": _traffic("gemm_smallm_decode_step", "hbm_bytes_per_step"),
                "algorithmic_bytes_per_step": gemm_bytes, "launches_per_step": g["launches"] // args.steps}
    step_bytes = gemm_bytes + 2 * B * N * cI + B * (2 * wd.k * c + 2 * wd.nh * c + 4 * wd.k)
    return {"workload": "decode_step_b8_ctx128k_d4096_bf16", "batch": B, "context": L, "d": d, "dc": dc,
            "us_per_step": round(ms * 1000, 3), "queries_per_s": round(B / (ms * 1e-3), 1),
            "step_hbm_fraction": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernels_us_per_step": {n: round(s_["total_ms"] / args.steps * 1000, 3) for n, s_ in kern.items()},
            "projection_roofline": roof, "input_copies": 2}


def cpu_baseline(dec, seconds):
    """The float64 oracle, as it stands, on whole queries of the same decode batch."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from compressed_sparse_attention_amd import synth
    from oracle import csa_oracle as O

    D, w = dec["D"], dec["workload"]
    scale = 1.0 / math.sqrt(w.c)
    done = 0
    t0 = time.perf_counter()
    while True:
        b = done % dec["B"]
        nc = int(D["seq_len"][b] // w.m)
        off = int(D["kv_offset"][b])
        K = synth.bf16_to_f64(D["KIcomp"][off:off + nc])
        s = O.index_scores_row(synth.bf16_to_f64(D["qI"][b]), D["wI"][b].astype(np.float64), K, nc)
        sel = O.topk(s, w.k)
        O.mqa(synth.bf16_to_f64(D["q"][b]), synth.bf16_to_f64(D["Ccomp"][off + sel]), scale)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(done / el, 3), "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} whole decode queries of the 8 x 131072-token batch (32768-key sweep, "
                      f"top-{w.k}, {w.nh}-head MQA each), float64 NumPy, {el:.1f} s"}


def calib_copy(torch):
    """A plain device copy of known size (for scaling memory counters)."""
    n = 1 << 28  # 2^28 fp32 = 1 GiB each way
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_each_way": 4 * n, "launches": 3}))


# the legs, by the name --only takes
_LEGS = {
    "decode": lambda a, t, api, sy, la: bench_decode(a, t, api, sy, la),
    "prefill": lambda a, t, api, sy, la: bench_prefill(a, t, api, sy, la, "dense"),
    "selection_long": lambda a, t, api, sy, la: bench_selection_long(a, t, api, sy, la),
    "decode_step": lambda a, t, api, sy, la: bench_decode_step(a, t, api, sy, la),
    "prefill_varlen": lambda a, t, api, sy, la: bench_prefill_varlen(a, t, api, sy, la),
    "prefill_backward": lambda a, t, api, sy, la: bench_prefill_backward(a, t, api, sy, la),
    "other_configs": lambda a, t, api, sy, la: bench_other_configs(a, t, api, sy, la),
}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--prefill-steps", type=int, default=3)
    ap.add_argument("--prefill-warmup", type=int, default=1)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-decode-step", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--only", choices=sorted(_LEGS), default=None,
                    help="run one leg on its own and print its record (for per-leg profiler traces)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the CSA path here is single-GPU "
              "(no sharding, no collectives); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calib_copy:
        calib_copy(torch)
        return
    from compressed_sparse_attention_amd import api, layer, synth
    api.lib()
    if args.only:
        rec = _LEGS[args.only](args, torch, api, synth, layer)
        if args.only == "decode":
            rec = {k: rec[k] for k in ("ms", "ms_eager", "ms_warm", "roofline", "step_bytes")} | {
                "kernels_us": {n: round(s_["avg_us"], 3) for n, s_ in rec["kernels"].items()}}
        elif args.only == "prefill":
            rec = rec[0]
        print(json.dumps({"only": args.only, "record": rec}, default=str), flush=True)
        return

    dec = bench_decode(args, torch, api, synth, layer)
    pre = pre_stream = sel_long = None
    if not args.no_prefill:
        pre, HW = bench_prefill(args, torch, api, synth, layer, "dense")
        pre_stream, HW = bench_prefill(args, torch, api, synth, layer, "stream", HW)
        del HW
        sel_long = bench_selection_long(args, torch, api, synth, layer)
    dstep = None if args.no_decode_step else bench_decode_step(args, torch, api, synth, layer)
    pvar = None if args.no_varlen else bench_prefill_varlen(args, torch, api, synth, layer)
    pbwd = None if args.no_backward else bench_prefill_backward(args, torch, api, synth, layer)
    other = None if args.no_other_configs else bench_other_configs(args, torch, api, synth, layer)
    cpu = None if args.no_cpu_baseline else cpu_baseline(dec, args.cpu_seconds)

    w = dec["workload"]
    # the step is timed both as HIP-graph replays and as eager launches; the
    # faster of the two is the reported rate (the other is on the line too)
    launch = "graph" if dec["ms"] <= dec["ms_eager"] else "eager"
    ms_step = min(dec["ms"], dec["ms_eager"])
    qps = dec["B"] / (ms_step * 1e-3)
    line = {
        "metric": "CSA decode queries/s at 128K ctx; prefill tokens/s; % HBM / MFMA roofline",
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; caches N(0,1), queries std dim^-1/2, head weights N(0,1))",
        "config": {"workload": w.name, "batch": dec["B"], "context": w.L, "m": w.m, "c": w.c, "cI": w.cI,
                   "nhI": w.nhI, "nh": w.nh, "k": w.k, "input_copies": args.replicas, "launch": launch},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "decode_step_hbm_fraction": round(dec["step_bytes"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "warm_cache_queries_per_s": round(dec["B"] / (dec["ms_warm"] * 1e-3), 1),
        "eager_queries_per_s": round(dec["B"] / (dec["ms_eager"] * 1e-3), 1),
        "graph_queries_per_s": round(dec["B"] / (dec["ms"] * 1e-3), 1),
        "step_time_stats": dec["dist"][launch],
        "step_time_stats_other_launch": dec["dist"]["eager" if launch == "graph" else "graph"],
        "decode_kernels_us": {n: round(s["avg_us"], 3) for n, s in dec["kernels"].items()},
        "prefill": pre,
        "prefill_stream_selection": pre_stream,
        "selection_long": sel_long,
        "decode_step_with_cache": dstep,
        "prefill_varlen": pvar,
        "prefill_backward": pbwd,
        "other_configs": other,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
