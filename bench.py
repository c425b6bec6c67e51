#!/usr/bin/env python3
"""Benchmark of paged decode attention on one MI355X.

One step = one decode step of a whole model's attention layers: for each of
`--layers` layers (each with its own K/V pool, so no layer's data can still be
in L2 / MALL when it is read) append one new token per sequence
(pa_reshape_and_cache) and run pa_decode over every sequence's paged context.

Default workload: Llama-2-7B-shaped decode -- 64 sequences, 32 q heads = 32 kv
heads x 128, fp16, block size 16, context lengths uniform in [1, 2048], pool =
needed blocks + 10 %, 32 layers.  Inputs are synthetic (seeded normal draws).

Prints ONE JSON line.  `value` is KV GB/s (bytes of K and V the decode calls
must read, over the whole timed region); the line also carries seq*layers/s,
the roofline of the decode call, and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
REPEATS = 5                 # back-to-back passes over all layers, for the median and the best
WARM_CALLS = 20             # decode calls on one layer's pool, for the warm (cached) figure
METRIC = "paged decode attention KV GB/s (% of HBM peak) and seq-layers/s, 1×MI355X"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: 3; 20 for the matrix-core bound prefill "
                         "and prefix_cache ops, whose clocks take that long to settle)")
    ap.add_argument("--workload", default="llama7b",
                    choices=["llama7b", "llama70b_gqa", "llama70b_tp8", "mixed_bs8", "mixed_bs16", "mixed_bs32",
                             "shared_prefix", "tiny_f32"])
    ap.add_argument("--layers", type=int, default=None, help="default: 32 (7B-shaped), 80 (70B-shaped)")
    ap.add_argument("--partition-tokens", type=int, default=None,
                    help="0 = library's choice (default), -1 = single pass, -2 = balanced schedule, N = split-K partition of N tokens")
    ap.add_argument("--layout", choices=["bhtd", "bthd"], default="bhtd")
    ap.add_argument("--shared-blocks", choices=["auto", "on", "off"], default="auto",
                    help="PA_DECODE_SHARED_BLOCKS: auto = on when the workload's tables share blocks")
    ap.add_argument("--prefix-pass", choices=["auto", "on", "off"], default="auto",
                    help="pa_decode_shared_prefix: auto = on when the workload's tables all start with the same blocks")
    ap.add_argument("--kernel", choices=["auto", "vector", "mfma"], default="auto",
                    help="decode kernel family (pa_kernel): auto picks matrix cores for grouped-query heads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time of the headline oracle samples (the other configurations get less)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the chosen workload, not the other configurations next to it")
    ap.add_argument("--config-steps", type=int, default=5, help="timed steps of each other configuration")
    ap.add_argument("--config-warmup", type=int, default=10,
                    help="untimed steps before each other configuration's timed ones (the clocks settle under load)")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read probe")
    ap.add_argument("--op", choices=["decode", "prefill", "prefix_cache", "copy_blocks", "swap_out", "swap_in"],
                    default="decode",
                    help="decode (the default step); prefill (a 512-token chunk per sequence over a 1536-token "
                         "cached history); or one of the block moves of the paging system: copy_blocks (copy on "
                         "write inside the GPU pools), swap_out / swap_in (GPU pools <-> pinned host pools)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device a few times (the known-size kernel that scales the "
                         "HBM byte counters of a profiler run) and exit")
    a = ap.parse_args(argv)
    if a.warmup is None:
        a.warmup = 20 if a.op in ("prefill", "prefix_cache") else 3
    return a


HOST_LINK_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense f16 / bf16 matrix-core peak of the MI355X


def prefix_cache_requests():
    """The 128 prompts: one 1504-token system prompt plus 8-200 tokens of each request's own."""
    S, sys_len, bs = 128, 1504, 16
    rng = np.random.default_rng(31)
    system = rng.integers(0, 32000, sys_len).astype(np.int32)
    own = rng.integers(8, 201, S)
    prompts = [np.concatenate([system, rng.integers(0, 32000, n).astype(np.int32)]) for n in own]
    NB = sum(-(-len(p) // bs) for p in prompts) + 16
    MB = max(-(-len(p) // bs) for p in prompts)
    return prompts, NB, MB, bs


def prefix_cache_admit(mgr, prompts, cached: bool):
    """Admit every request into a block manager (the library's or the model), in order; returns the cache hits."""
    hits = []
    for sid, p in enumerate(prompts):
        hit = mgr.add_cached(sid, p) if cached else (mgr.add(sid) or 0)
        mgr.append_tokens(sid, p[hit:])
        hits.append(hit)
    return hits


def prefix_cache_measure(torch, B, steps, warmup, host_reps=1):
    """The GPU prefill of the 127 requests admitted after the first: with the cache and the shared-prefix call
    ("cached"), with the cache and pa_prefill per request ("cached_plain"), without the cache ("full");
    each call timed back to back between one pair of events.  Also the library manager's admission time."""
    S, H, D = 128, 32, 128
    prompts, NB, MB, bs = prefix_cache_requests()
    dev = torch.device("cuda:0")
    # host: admitting every request (the first computes its prompt, the rest hit the cache)
    t = time.perf_counter()
    for _ in range(host_reps):
        bm = B.BlockManager(NB, 0, bs)
        hits = prefix_cache_admit(bm, prompts, True)
        tables_c, lens_c = bm.block_tables(list(range(S)), MB)
        bm.close()
    host_us = (time.perf_counter() - t) / host_reps / S * 1e6
    bm = B.BlockManager(NB, 0, bs)
    prefix_cache_admit(bm, prompts, False)
    tables_f, lens_f = bm.block_tables(list(range(S)), MB)
    bm.close()

    gen = torch.Generator(device=dev)
    gen.manual_seed(32)
    kc = torch.randn((NB, H, bs, D), generator=gen, device=dev, dtype=torch.float16)
    vc = torch.randn_like(kc)
    scale = float(np.float32(1 / np.sqrt(D)))
    stream = torch.cuda.current_stream()
    later = list(range(1, S))                       # the requests admitted after the first

    def batch(tables, lens, hits_):
        rows = [len(prompts[i]) - hits_[i] for i in later]
        qs = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
        q = torch.randn((int(qs[-1]), H, D), generator=gen, device=dev, dtype=torch.float16)
        return (q, torch.empty_like(q), torch.from_numpy(tables[later]).to(dev), torch.from_numpy(lens[later]).to(dev),
                torch.from_numpy(qs).to(dev), max(rows), rows)

    runs = {"cached": batch(tables_c, lens_c, hits), "full": batch(tables_f, lens_f, [0] * S)}
    runs["cached_plain"] = runs["cached"]
    # the blocks every admitted request shares from the cache (the system prompt's): read once for all their rows
    prefix_blocks = min(hits[i] for i in later) // bs
    q_c = runs["cached"][0]
    ws = torch.empty(max(1, B.pa_prefill_shared_prefix_workspace_bytes(q_c.shape[0], H, D, bs, prefix_blocks)),
                     dtype=torch.uint8, device=dev)

    def call(r):
        q, out, t_dev, l_dev, qs_dev, mq, _ = runs[r]
        if r == "cached":
            B.pa_prefill_shared_prefix(out, q, kc, vc, t_dev, l_dev, qs_dev, mq, scale, prefix_blocks, num_blocks=NB,
                                       workspace=ws, stream=stream)
        else:
            B.pa_prefill(out, q, kc, vc, t_dev, l_dev, qs_dev, mq, scale, num_blocks=NB, stream=stream)

    ms = {}
    for r in runs:
        for _ in range(warmup):
            call(r)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            call(r)
        t1.record(stream)
        torch.cuda.synchronize()
        ms[r] = t0.elapsed_time(t1) / steps
    del runs, kc, vc, ws
    prompt_tokens = sum(len(prompts[i]) for i in later)
    # algorithmic flops of the cached call: each computed row attends its position + 1 tokens
    flops = sum(sum(hits[i] + j + 1 for j in range(len(prompts[i]) - hits[i])) for i in later) * H * 4 * D
    return {"ms": ms, "flops": flops, "achieved": flops / (ms["cached"] * 1e-3) / 1e12, "hits": hits,
            "prompt_tokens": prompt_tokens, "tokens_from_cache": sum(hits[i] for i in later),
            "prefix_blocks": prefix_blocks, "host_us": host_us}


def prefix_cache_step(args):
    """Automatic prefix caching on the pages' customer-service case, at the shared-prefix workload's scale:
    128 requests whose prompts are one 1504-token system prompt plus 8-200 tokens of their own (32 x 128 MHA
    heads, fp16, block size 16).  The first request computes its whole prompt; then the other 127 are
    admitted and prefilled, with the cache (the library's block manager: they reuse the 94 system-prompt
    blocks and compute only their own tokens; pa_prefill_shared_prefix reads those blocks once for all of
    their rows, pa_prefill per request is timed beside it) and without it (every prompt computed in full).  Host: the
    library's manager admitting a request (pa_bm_add_cached + pa_bm_append_tokens), the oracle's model
    beside it."""
    import torch
    from paged_kv_cache_405_amd import binding as B
    from oracle.prefix_cache import PrefixCacheModel
    torch.cuda.set_device(torch.device("cuda:0"))
    B.lib()
    m = prefix_cache_measure(torch, B, args.steps, args.warmup, host_reps=max(1, args.steps // 5))
    ms, hits, host_us, prefix_blocks = m["ms"], m["hits"], m["host_us"], m["prefix_blocks"]
    S = len(hits)
    prompts, NB, _, bs = prefix_cache_requests()
    t = time.perf_counter()
    model = PrefixCacheModel(NB, 0, bs)
    mhits = prefix_cache_admit(model, prompts, True)        # the model on the same int32 token arrays
    model_us = (time.perf_counter() - t) / S * 1e6
    assert mhits == hits, "the library and the model disagree on the cache hits"
    log(f"[bench] prefix cache: {sum(h > 0 for h in hits)} of {S} requests hit, {hits[1]} tokens each; "
        f"host {host_us:.2f} us per request (library), {model_us:.1f} us (oracle model)")
    log(f"[bench] prefill of 127 admitted requests: {ms['cached'] * 1e3:.1f} us with the cache "
        f"({prefix_blocks} shared blocks read once for all rows; {ms['cached_plain'] * 1e3:.1f} us with pa_prefill), "
        f"{ms['full'] * 1e3:.1f} us without ({ms['full'] / ms['cached']:.1f}x)")
    prompt_tokens = m["prompt_tokens"]
    result = {
        "metric": "prompt tokens made ready per second with automatic prefix caching (GPU prefill)",
        "value": round(prompt_tokens / (ms["cached"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms["cached"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded token ids, K/V, q)",
        "config": {"workload": "prefix_cache: 128 requests, 1504-token shared system prompt + 8-200 own tokens, "
                               "32x128 MHA, fp16, block size 16; prefill of the 127 requests after the first",
                   "parallelism": "single GPU"},
        "prefill_us_with_cache": round(ms["cached"] * 1e3, 2),
        "prefill_us_with_cache_per_request": round(ms["cached_plain"] * 1e3, 2),
        "shared_prefix_blocks": prefix_blocks,
        "prefill_us_without_cache": round(ms["full"] * 1e3, 2),
        "speedup": round(ms["full"] / ms["cached"], 2),
        "prompt_tokens_from_cache": round(m["tokens_from_cache"] / prompt_tokens, 4),
        "host_us_per_request": round(host_us, 3),
        "roofline": {"kernel": "prefill_wide_kernel (the cached call: the shared prefix once for every row, then "
                               "each request's own keys)", "bound": "mfma", "achieved": round(m["achieved"], 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(m["achieved"] / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": None, "avg_call_us": round(ms["cached"] * 1e3, 3), "flops_per_call": m["flops"]},
        "cpu_baseline": {"value": round(1e6 / model_us, 1), "unit": "requests admitted/s", "cores": 1,
                         "kind": "oracle", "sample": "the prefix-cache model admitting the same 128 requests "
                                                     f"({model_us:.1f} us each; the library: {host_us:.2f} us)"},
    }
    print(json.dumps(result), flush=True)


PREFILL_SHAPE = dict(S=16, chunk=512, hist=1536, H=32, D=128, bs=16)


def prefill_measure(torch, B, steps, warmup, layers):
    """pa_prefill on Llama-2-7B-shaped layers, the calls back to back between one pair of events: 16 sequences,
    each attending a 512-token chunk over a 1536-token cached history (context 2048), 32 x 128 MHA heads, fp16,
    block size 16, `layers` layers with their own pools."""
    S, chunk, hist, H, D, bs = (PREFILL_SHAPE[k] for k in ("S", "chunk", "hist", "H", "D", "bs"))
    dev = torch.device("cuda:0")
    ctx = hist + chunk
    nblk = ctx // bs
    NB = S * nblk + S * nblk // 10
    rng = np.random.default_rng(21)
    # distinct blocks for every sequence: one permutation of the pool
    perm = rng.permutation(NB)
    tables = perm[:S * nblk].reshape(S, nblk).astype(np.int32)
    gen = torch.Generator(device=dev)
    gen.manual_seed(22)
    Ls = []
    for _ in range(layers):
        kc = torch.randn((NB, H, bs, D), generator=gen, device=dev, dtype=torch.float16)
        vc = torch.randn_like(kc)
        q = torch.randn((S * chunk, H, D), generator=gen, device=dev, dtype=torch.float16)
        Ls.append((kc, vc, q, torch.empty_like(q)))
    t_dev = torch.from_numpy(tables).to(dev)
    ctx_dev = torch.full((S,), ctx, dtype=torch.int32, device=dev)
    qs_dev = torch.arange(0, S * chunk + 1, chunk, dtype=torch.int32, device=dev)
    scale = float(np.float32(1 / np.sqrt(D)))
    stream = torch.cuda.current_stream()

    def step():
        for kc, vc, q, out in Ls:
            B.pa_prefill(out, q, kc, vc, t_dev, ctx_dev, qs_dev, chunk, scale, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for k in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    call_ms = total_ms / (steps * layers)
    # algorithmic work: query row i of a chunk attends hist + i + 1 tokens; 2 D flops for q.k and 2 D for p.v
    attended = S * sum(hist + i + 1 for i in range(chunk))
    flops = attended * H * 4 * D
    del Ls
    return {"total_ms": total_ms, "call_ms": call_ms, "flops": flops, "layers": layers, "steps": steps,
            "achieved": flops / (call_ms * 1e-3) / 1e12}


def prefill_step(args):
    """Time chunked prefill (pa_prefill) on Llama-2-7B-shaped layers: 16 sequences, each appending and
    attending a 512-token chunk over a 1536-token cached history (context 2048), 32 x 128 MHA heads, fp16,
    block size 16; 8 layers with their own pools."""
    import torch
    from paged_kv_cache_405_amd import binding as B
    from oracle.prefill import paged_prefill
    torch.cuda.set_device(torch.device("cuda:0"))
    B.lib()
    S, chunk, hist, H, D, bs = (PREFILL_SHAPE[k] for k in ("S", "chunk", "hist", "H", "D", "bs"))
    ctx = hist + chunk
    nblk = ctx // bs
    layers = args.layers or 8
    m = prefill_measure(torch, B, args.steps, args.warmup, layers)
    total_ms, call_ms, flops, achieved = m["total_ms"], m["call_ms"], m["flops"], m["achieved"]
    calls = args.steps * layers
    scale = float(np.float32(1 / np.sqrt(D)))
    # the oracle, as it is, on one sequence of the same shape (K/V drawn on the host)
    rng = np.random.default_rng(23)
    hk = fp16_storage(rng.standard_normal((nblk, bs, H, D), dtype=np.float32))
    hv = fp16_storage(rng.standard_normal((nblk, bs, H, D), dtype=np.float32))
    hq = fp16_storage(rng.standard_normal((chunk, H, D), dtype=np.float32))
    t = time.perf_counter()
    paged_prefill(hq, hk, hv, np.arange(nblk, dtype=np.int32)[None], np.array([ctx], np.int32),
                  np.array([0, chunk], np.int32), scale, "f16")
    cpu_s = time.perf_counter() - t
    result = {
        "metric": "paged prefill TFLOP/s (causal chunk over a paged history), 1xMI355X",
        "value": round(flops * calls / (total_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic (normal draws)",
        "config": {"workload": f"prefill: {S} seqs x {chunk}-token chunk over {hist} cached tokens, {H}x{D} MHA, "
                               f"fp16, bs {bs}, {layers} layers", "chunk": chunk, "history": hist},
        "roofline": {"kernel": "prefill_wide_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": None, "avg_call_us": round(call_ms * 1e3, 3), "flops_per_call": flops},
        "cpu_baseline": {"value": round(flops / S / cpu_s / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                         "sample": f"one sequence of the same shape ({chunk} rows over {ctx} tokens), fp64 numpy"},
    }
    print(json.dumps(result), flush=True)


def fp16_storage(x32):
    """fp32 draws rounded to fp16 storage."""
    return x32.astype(np.float16)


def block_moves(args):
    """Time one of the block moves on Llama-2-7B-shaped blocks (32 kv heads x 16 tokens x 128, fp16:
    128 KiB of K and of V per block): copy on write of 1024 blocks inside 8192-block GPU pools, or
    swapping 256 blocks between those pools and 2048-block pinned host pools."""
    import torch
    from paged_kv_cache_405_amd import binding as B
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()
    bs, Hkv, D = 16, 32, 128
    NG, NC = 8192, 2048
    n = 1024 if args.op == "copy_blocks" else 256
    block_bytes = bs * Hkv * D * 2
    rng = np.random.default_rng(11)
    gk = torch.randn((NG, Hkv, bs, D), device=dev, dtype=torch.float16)
    gv = torch.randn_like(gk)
    if args.op == "copy_blocks":
        perm = rng.permutation(NG)
        pairs = np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int32)
        ck = cv = None
    else:
        ck = torch.empty((NC, Hkv, bs, D), dtype=torch.float16).pin_memory()
        cv = torch.empty_like(ck).pin_memory()
        ck.normal_()
        cv.normal_()
        g, c = rng.permutation(NG)[:n], rng.permutation(NC)[:n]
        pairs = np.stack([g, c] if args.op == "swap_out" else [c, g], 1).astype(np.int32)
    dpairs = torch.from_numpy(pairs).to(dev)
    stream = torch.cuda.current_stream()

    def call():
        if args.op == "copy_blocks":
            B.copy_blocks(gk, gv, dpairs, stream=stream)
        elif args.op == "swap_out":
            B.swap_blocks(ck, cv, gk, gv, dpairs, stream=stream)
        else:
            B.swap_blocks(gk, gv, ck, cv, dpairs, stream=stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # the calls back to back between one pair of events
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    call_ms = total_ms / args.steps
    moved = 2 * n * block_bytes                      # K and V blocks
    if args.op == "copy_blocks":
        bound, peak, algo = "hbm", HBM_PEAK_GBS, 2 * moved     # read and write, both in HBM
    else:
        bound, peak, algo = "host-link", HOST_LINK_PEAK_GBS, moved   # each byte crosses the link once
    achieved = algo / (call_ms * 1e-3) / 1e9
    # the oracle's copy (numpy, as it is) on a bounded sample of the same blocks
    from oracle.blocks import copy_blocks as oracle_copy
    sample = 64
    hk = np.random.default_rng(1).standard_normal((sample * 2, Hkv, bs, D)).astype(np.float16)
    hv = hk.copy()
    sp = np.stack([np.arange(sample), np.arange(sample, 2 * sample)], 1)
    t = time.perf_counter()
    reps = 0
    while time.perf_counter() - t < min(args.cpu_seconds, 5.0) or reps == 0:
        oracle_copy(hk, hv, sp)
        reps += 1
    cpu_s = time.perf_counter() - t
    result = {
        "metric": f"{args.op} GB/s (K and V blocks moved), 1xMI355X",
        "value": round(algo * args.steps / (total_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic (normal draws)",
        "config": {"workload": f"{args.op}: {n} blocks of 32 kv heads x 16 tokens x 128 fp16 (128 KiB of K and "
                               f"of V each), GPU pools of {NG} blocks, pinned host pools of {NC}",
                   "pairs": n, "block_bytes": block_bytes},
        "roofline": {"kernel": "copy_blocks_kernel", "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": "GB/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "avg_call_us": round(call_ms * 1e3, 3), "bytes_per_call": algo},
        "cpu_baseline": {"value": round(2 * 2 * sample * block_bytes * reps / cpu_s / 1e9, 3), "unit": "GB/s",
                         "cores": 1, "kind": "oracle",
                         "sample": f"{reps} numpy copies of {sample} block pairs (K and V), one thread"},
    }
    print(json.dumps(result), flush=True)


def copy_calibration():
    """A plain device copy of known size: each dispatch reads and writes exactly 1 GiB."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_dispatch": n, "bytes_written_per_dispatch": n,
                                           "dispatches": 3}}), flush=True)


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_sample(w, target_s, seqs_start=0):
    """One timing of the CPU oracle (as it is) on a bounded sample of the workload: whole sequences of
    layer 0, as many as fit in about target_s seconds.  Returns (seconds, K/V bytes, sequences)."""
    import oracle
    S = w.num_seqs
    n = max(1, min(S, 4))
    elapsed, nbytes, nseq, reps = 0.0, 0, 0, 0
    idx = seqs_start % S
    while elapsed < target_s and reps < 64:
        sel = [(idx + i) % S for i in range(n)]
        idx = (idx + n) % S
        cl = w.context_lens[sel]
        t0 = time.perf_counter()
        oracle.paged_decode(w.q[sel], w.k_cache, w.v_cache, w.block_tables[sel], cl, w.scale, w.dtype)
        dt = time.perf_counter() - t0
        elapsed += dt
        nbytes += int(np.sum(cl.astype(np.int64))) * w.num_kv_heads * 2 * w.head_dim * w.elem_bytes
        nseq += n
        reps += 1
        if dt > 0 and elapsed < target_s:
            n = int(min(S, max(1, n * max(1.0, (target_s - elapsed) / dt / 2))))
    return elapsed, nbytes, nseq


def cpu_rates(w, target_s, runs=3):
    """The oracle's median rate over `runs` bounded samples (each about target_s seconds)."""
    import oracle
    samples = [cpu_sample(w, target_s, seqs_start=17 * r) for r in range(runs)]
    gbs = [b / t / 1e9 for t, b, _ in samples]
    sps = [n / t for t, _, n in samples]
    return {
        "value": round(statistics.median(gbs), 4), "unit": "GB/s",
        "seq_layers_per_s": round(statistics.median(sps), 2),
        "runs": runs, "values": [round(x, 4) for x in gbs],
        "seconds": round(sum(t for t, _, _ in samples), 3),
        "threads": oracle.num_threads(),
        "sample": f"{sum(n for _, _, n in samples)} sequence-layers over {runs} samples",
    }


def cpu_baseline_one_core(name, target_s, runs=3):
    """The same oracle samples on one host core: a child process with OMP_NUM_THREADS=1."""
    import subprocess
    code = ("import json, sys; sys.path.insert(0, %r); import bench; from paged_kv_cache_405_amd import workloads as W; "
            "r = bench.cpu_rates(W.WORKLOADS[%r](poison=False), %r, %d); print(json.dumps(r))"
            % (os.path.dirname(os.path.abspath(__file__)), name, float(target_s), runs))
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"one-core oracle sample failed: {r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def cpu_baseline(args, w):
    """The CPU oracle (fp64 C, OpenMP over sequences and heads, as it is) on the GPU machine's host cores, on
    bounded samples of the headline workload: median of 3 samples with all threads, and with one thread."""
    t = args.cpu_seconds
    main = cpu_rates(w, t / 3)
    res = {
        "value": main["value"], "unit": "GB/s", "cores": main["threads"], "kind": "oracle",
        "sample": (f"{main['sample']} of the {w.name} workload (whole sequences, all q heads, fp64), median of "
                   f"{main['runs']}; {main['threads']} OpenMP threads; {len(os.sched_getaffinity(0))} host cores in "
                   f"the affinity mask; CPU: {cpu_model()}"),
        "seq_layers_per_s": main["seq_layers_per_s"], "values": main["values"], "seconds": main["seconds"],
        "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
    }
    res["one_core"] = cpu_baseline_one_core(w.name, t / 6)
    return res


# the configurations reported next to the headline workload (the five workloads, the mixed batch at every
# block size); each runs with its own pools, freed before the next one
CONFIG_WORKLOADS = ["tiny_f32", "llama7b", "mixed_bs8", "mixed_bs16", "mixed_bs32", "shared_prefix",
                    "llama70b_gqa"]
CONFIG_POOL_BYTES = 40e9    # each config rotates over its model's layers, as many as fit in this many bytes of pools


def run_config(args, w, B):
    """The host-side settings of a run (no device needed)."""
    return {
        "layers": args.layers or (80 if w.name.startswith("llama70b") else 32),
        "layout": B.PA_LAYOUT_BHTD if args.layout == "bhtd" else B.PA_LAYOUT_BTHD,
        # the library's own choice unless a partition is asked for
        "pt": B.PA_PARTITION_AUTO if args.partition_tokens is None else args.partition_tokens,
        "kern": {"auto": B.PA_KERNEL_AUTO, "vector": B.PA_KERNEL_VECTOR, "mfma": B.PA_KERNEL_MFMA}[args.kernel],
        "dtype_code": {"f32": B.PA_F32, "f16": B.PA_F16, "bf16": B.PA_BF16}[w.dtype],
        # the caller knows when several sequences read the same blocks (a shared prefix)
        "shared": args.shared_blocks == "on" or (args.shared_blocks == "auto" and w.shared_prefix_blocks > 0),
        # ... and can then name the prefix, read once for the whole batch
        "prefix_pass": w.shared_prefix_blocks > 0 and (args.prefix_pass == "on" or args.prefix_pass == "auto"),
    }


def decode_run(args, w, cfg, layers, steps, warmup, torch, B, repeats=REPEATS, warm_calls=WARM_CALLS):
    """Time one workload: `layers` layers with their own pools; a step appends one token per sequence and
    decodes, layer by layer.  Returns the measurements (no JSON formatting)."""
    dev = torch.device("cuda:0")
    layout, pt, kern, shared, dtype_code = (cfg[k] for k in ("layout", "pt", "kern", "shared", "dtype_code"))
    prefix_pass = cfg["prefix_pass"]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]

    def dev_arr(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # layer 0 holds the seeded workload; the other layers get their own pools
    # and queries from a seeded device generator (same shapes, same tables)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    tables = torch.from_numpy(w.block_tables).to(dev)
    ctx = torch.from_numpy(w.context_lens).to(dev)
    slots = torch.from_numpy(w.slot_mapping).to(dev)
    kc0 = B.to_layout(dev_arr(w.k_cache), layout)
    cache_shape = tuple(kc0.shape)
    Ls = []
    for li in range(layers):
        if li == 0:
            kc, vc = kc0, B.to_layout(dev_arr(w.v_cache), layout)
            q, nk, nv = dev_arr(w.q), dev_arr(w.new_k), dev_arr(w.new_v)
        else:
            kc = torch.randn(cache_shape, generator=gen, device=dev, dtype=tdt)
            vc = torch.randn(cache_shape, generator=gen, device=dev, dtype=tdt)
            q = torch.randn(tuple(w.q.shape), generator=gen, device=dev, dtype=tdt)
            nk = torch.randn(tuple(w.new_k.shape), generator=gen, device=dev, dtype=tdt)
            nv = torch.randn(tuple(w.new_v.shape), generator=gen, device=dev, dtype=tdt)
        Ls.append((kc, vc, q, nk, nv, torch.empty_like(q)))
    if prefix_pass:
        ws_bytes = B.pa_decode_shared_prefix_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                                             w.block_size, w.max_blocks_per_seq, dtype_code,
                                                             w.shared_prefix_blocks)
    else:
        ws_bytes = B.pa_decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                               w.max_blocks_per_seq, dtype_code, pt)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    kv_per_layer = w.kv_bytes()
    log(f"[bench] {w.name}: pools ready: {layers} x {2 * kc0.numel() * kc0.element_size() / 1e9:.2f} GB; "
        f"KV bytes per decode call {kv_per_layer / 1e9:.4f} GB; workspace {ws_bytes} B")

    stream = torch.cuda.current_stream()
    # the path the library resolves the automatic choices to
    path_pt, path_kern = B.pa_decode_path(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                          w.max_blocks_per_seq, dtype_code, pt, kern)
    family = "mfma" if path_kern == B.PA_KERNEL_MFMA else "vec"
    if path_pt == B.PA_PARTITION_BALANCED:
        path_name, call_kernels = "balanced", f"decode_stream_kernel ({family}) + stream_reduce_kernel"
    elif path_pt == B.PA_PARTITION_SINGLE:
        path_name, call_kernels = "single", f"decode_{family}_kernel"
    else:
        path_name, call_kernels = f"split-K {path_pt} tokens", f"decode_{family}_kernel + reduce_kernel"
    if prefix_pass:
        path_name = f"shared prefix ({w.shared_prefix_blocks} blocks) once, then split-K"
        # the library runs both passes in one launch when the own blocks take the vector kernel
        call_kernels = ("shared_prefix_kernel (the prefix pass beside the sequences' own blocks) + reduce_kernel"
                        if family == "vec" else
                        f"prefix_kernel + decode_{family}_kernel (the sequences' own blocks) + reduce_kernel")
    log(f"[bench] {w.name}: path {path_name}, kernels per call: {call_kernels}")

    def decode(out, q, kc, vc):
        if prefix_pass:
            B.pa_decode_shared_prefix(out, q, kc, vc, tables, ctx, w.scale, w.shared_prefix_blocks, layout=layout,
                                      workspace=ws, stream=stream)
        else:
            B.pa_decode_ex(out, q, kc, vc, tables, ctx, w.scale, layout=layout, partition_tokens=pt,
                           kernel=kern, shared_blocks=shared, workspace=ws, stream=stream)

    def step(events=None):
        for li, (kc, vc, q, nk, nv, out) in enumerate(Ls):
            B.pa_reshape_and_cache(nk, nv, kc, vc, slots, layout=layout, stream=stream)
            if events is not None:
                events[2 * li].record(stream)
            decode(out, q, kc, vc)
            if events is not None:
                events[2 * li + 1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * layers)] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(steps):
        step(ev[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    call_ms = [ev[k][2 * li].elapsed_time(ev[k][2 * li + 1]) for k in range(steps) for li in range(layers)]
    evented_call_ms = statistics.fmean(call_ms)
    # the launch duration of a decode call: the same calls back to back, one
    # event pair around all of them (an event pair per call adds its own
    # few microseconds to every call it brackets)
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for k in range(steps):
        for kc, vc, q, nk, nv, out in Ls:
            decode(out, q, kc, vc)
    d1.record(stream)
    torch.cuda.synchronize()
    avg_call_ms = d0.elapsed_time(d1) / (steps * layers)
    log(f"[bench] {w.name}: {steps} steps {total_ms:.3f} ms; decode calls back to back {avg_call_ms * 1e3:.2f} us "
        f"per call (between their own events {evented_call_ms * 1e3:.2f} us)")

    def back_to_back(fn, n):
        """Average duration of n calls of fn() issued back to back between one event pair."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def all_layers(fn):
        return lambda: [fn(*L) for L in Ls]

    # the same back-to-back pass over every layer, repeated: median and best
    reps = [back_to_back(all_layers(lambda kc, vc, q, nk, nv, out: decode(out, q, kc, vc)), 1) / layers
            for _ in range(repeats)]
    # the append kernel alone, every layer once per pass
    append_us = back_to_back(all_layers(lambda kc, vc, q, nk, nv, out: B.pa_reshape_and_cache(
        nk, nv, kc, vc, slots, layout=layout, stream=stream)), steps) / layers
    # warm: layer 0's pool again and again (it can then sit in the caches: not a decode step);
    # few calls, so that a kernel trace's average over the run stays that of the real step
    kc, vc, q, _, _, out = Ls[0]
    warm_us = back_to_back(lambda: decode(out, q, kc, vc), warm_calls)
    log(f"[bench] {w.name}: back-to-back passes median {statistics.median(reps):.2f} us, best {min(reps):.2f} us; "
        f"append alone {append_us:.2f} us; warm same pool {warm_us:.2f} us")

    # the bytes a call must read: every token's K and V once -- with the prefix
    # pass, the shared prefix once for the whole batch
    roof_bytes = kv_per_layer
    if prefix_pass:
        pre = w.shared_prefix_blocks * w.block_size
        own = np.maximum(w.context_lens.astype(np.int64) - pre, 0).sum()
        roof_bytes = int((pre + own) * w.num_kv_heads * w.head_dim * w.k_cache.dtype.itemsize * 2)
    from paged_kv_cache_405_amd import traffic as TR
    rec = TR.lookup(w.name, path_pt, path_kern, args.layout, shared, prefix_pass=prefix_pass)
    del Ls, ws, kc0, kc, vc, q, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {
        "layers": layers, "steps": steps, "warmup": warmup, "total_ms": total_ms, "avg_call_ms": avg_call_ms,
        "evented_call_ms": evented_call_ms, "reps": reps, "append_us": append_us, "warm_us": warm_us,
        "path_name": path_name, "call_kernels": call_kernels, "family": family, "kv_per_layer": kv_per_layer,
        "roof_bytes": roof_bytes, "traffic_record": rec,
    }


def stream_probe(torch, B, nbytes=8 << 30, reps=3):
    """The streaming-read probe (pa_probe_stream_read) on an 8 GiB buffer: the best read rate over a few
    workgroup counts of the contiguous and grid-stride modes, and the rate of the scattered 4 KiB block mode
    (a paged pool's access pattern), each timed back to back (reps launches between one event pair).
    Context for the HBM fraction of the decode kernels; the roofline's peak stays 8 TB/s."""
    dev = torch.device("cuda:0")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    results = []
    for mode, wgs in ((0, 1024), (0, 2048), (0, 4096), (0, 8192), (1, 2048), (1, 8192), (2, 2048), (2, 8192)):
        B.pa_probe_stream_read(buf, sink, wgs, mode, stream=stream)          # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            B.pa_probe_stream_read(buf, sink, wgs, mode, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        results.append({"mode": ["contiguous chunk per workgroup", "grid stride", "scattered 4 KiB blocks"][mode],
                        "workgroups": wgs, "us": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)})
    del buf, sink
    torch.cuda.empty_cache()
    best = max((r for r in results if r["mode"] != "scattered 4 KiB blocks"), key=lambda r: r["gbs"])
    log(f"[bench] streaming-read probe: best {best['gbs']} GB/s ({best['mode']}, {best['workgroups']} workgroups)")
    return best, results


def config_entry(w, m, traffic_ok=True):
    """The measurements of one workload as a JSON object."""
    achieved = m["roof_bytes"] / (m["avg_call_ms"] * 1e-3) / 1e9
    calls = m["steps"] * m["layers"]
    rec = m["traffic_record"]
    return {
        "workload": f"{w.name}: {w.description}", "dtype": w.dtype, "layers": m["layers"], "steps": m["steps"],
        "path": m["path_name"], "kernels": m["call_kernels"],
        "call_us": round(m["avg_call_ms"] * 1e3, 3),
        "call_us_repeats_median": round(statistics.median(m["reps"]), 3),
        "bytes_per_call": m["roof_bytes"], "achieved_gbs": round(achieved, 2),
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": None if rec is None or not traffic_ok else int(round(rec["bytes_per_call"])),
        "seq_layers_per_s": round(w.num_seqs * calls / (m["total_ms"] * 1e-3), 1),
        "append_and_decode_us_per_layer": round(m["total_ms"] * 1e3 / calls, 3),
        "kv_gbs_step": round(m["kv_per_layer"] * calls / (m["total_ms"] * 1e-3) / 1e9, 2),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_cache_405_amd import binding as B
    from paged_kv_cache_405_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.op == "prefill":
        prefill_step(args)
        return
    if args.op == "prefix_cache":
        prefix_cache_step(args)
        return
    if args.op != "decode":
        block_moves(args)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()                                                    # fail loudly if the library is missing

    w = W.WORKLOADS[args.workload](poison=False)
    cfg = run_config(args, w, B)
    log(f"[bench] workload {w.name}: {w.description}; layers {cfg['layers']}; partition {cfg['pt']}; "
        f"layout {args.layout}")
    m = decode_run(args, w, cfg, cfg["layers"], args.steps, args.warmup, torch, B)
    calls = args.steps * m["layers"]
    total_ms, avg_call_ms = m["total_ms"], m["avg_call_ms"]
    kv_gbs = m["kv_per_layer"] * calls / (total_ms * 1e-3) / 1e9
    achieved = m["roof_bytes"] / (avg_call_ms * 1e-3) / 1e9
    rec = m["traffic_record"]
    result = {
        "metric": METRIC,
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal q/K/V, seeded block tables and context lengths)",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "layers": m["layers"],
            "partition_tokens": cfg["pt"], "layout": args.layout, "kernel": args.kernel,
            "path": {"partition": m["path_name"], "kernel_family": m["family"]},
            "shared_blocks": cfg["shared"], "prefix_pass": cfg["prefix_pass"],
            "sum_context_tokens": int(w.context_lens.sum()), "parallelism": "single GPU",
        },
        "seq_layers_per_s": round(w.num_seqs * calls / (total_ms * 1e-3), 1),
        "hbm_peak_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "kv_bytes_per_layer": m["kv_per_layer"],
        "roofline": {
            "kernel": f"pa_decode call: {m['call_kernels']}",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if rec is None else int(round(rec["bytes_per_call"])),
            "traffic_source": None if rec is None else "profiles/hbm_traffic.json (rocprofv3 FETCH_SIZE, WRITE_SIZE)",
            "avg_call_us": round(avg_call_ms * 1e3, 3),
            "avg_call_us_own_events": round(m["evented_call_ms"] * 1e3, 3),
            "bytes_per_call": m["roof_bytes"],
        },
        "append_and_decode_us_per_layer": round(total_ms * 1e3 / calls, 3),
        "append_us": round(m["append_us"], 3),
        "call_us_repeats": {"n": REPEATS, "median": round(statistics.median(m["reps"]), 3),
                            "best": round(min(m["reps"]), 3),
                            "what": "all layers' decode calls back to back, one event pair per pass"},
        "warm_same_pool_call_us": round(m["warm_us"], 3),
    }
    if not args.no_probe:
        best, allp = stream_probe(torch, B)
        result["roofline"]["stream_probe_gbs"] = best["gbs"]
        result["roofline"]["scattered_4k_probe_gbs"] = max(r["gbs"] for r in allp if r["mode"] == "scattered 4 KiB blocks")
        result["roofline"]["stream_probe"] = {"best": best, "all": allp,
                                              "what": "pa_probe_stream_read over 8 GiB, non-temporal 16-byte loads"}
    if not args.no_configs:
        # the other configurations, each with its own pools (freed before the next)
        configs = {}
        for name in CONFIG_WORKLOADS:
            if name == w.name:
                continue
            cw = W.WORKLOADS[name](poison=False)
            ccfg = run_config(args, cw, B)
            pool = 2 * cw.k_cache.nbytes
            layers = max(4, min(ccfg["layers"], int(np.ceil(CONFIG_POOL_BYTES / max(pool, 1)))))
            cm = decode_run(args, cw, ccfg, layers, args.config_steps, args.config_warmup, torch, B, repeats=3, warm_calls=5)
            configs[name] = config_entry(cw, cm)
            if not args.no_cpu_baseline:
                # the oracle on the same workload: median of 3 shorter samples, all threads
                r = cpu_rates(cw, args.cpu_seconds / 8)
                configs[name]["cpu_baseline"] = {k: r[k] for k in ("value", "unit", "seq_layers_per_s", "values",
                                                                   "seconds", "threads")}
            del cw
        # the multi-token calls at their benchmarked shapes (matrix-core bound: TFLOP/s against the f16 peak)
        pm = prefill_measure(torch, B, max(10, args.config_steps), max(20, args.config_warmup), 8)
        configs["prefill_7b_chunk512"] = {
            "workload": "pa_prefill: 16 seqs x 512-token chunk over 1536 cached tokens, 32x128 MHA, fp16, bs 16",
            "kernel": "prefill_wide_kernel", "layers": pm["layers"], "steps": pm["steps"],
            "call_us": round(pm["call_ms"] * 1e3, 3), "flops_per_call": pm["flops"],
            "achieved_tflops": round(pm["achieved"], 2), "peak_tflops": MFMA_F16_PEAK_TFLOPS,
            "frac": round(pm["achieved"] / MFMA_F16_PEAK_TFLOPS, 4)}
        cm = prefix_cache_measure(torch, B, max(10, args.config_steps), max(20, args.config_warmup))
        configs["prefix_cache"] = {
            "workload": "pa_prefill_shared_prefix: the 127 requests admitted after the first onto a cached 1504-token "
                        "system prompt (8-200 own tokens each), 32x128 MHA, fp16, bs 16",
            "kernel": "prefill_wide_kernel (own pass, then the shared-prefix pass)", "steps": max(10, args.config_steps),
            "call_us": round(cm["ms"]["cached"] * 1e3, 3),
            "call_us_pa_prefill_per_request": round(cm["ms"]["cached_plain"] * 1e3, 3),
            "call_us_without_cache": round(cm["ms"]["full"] * 1e3, 3), "flops_per_call": cm["flops"],
            "achieved_tflops": round(cm["achieved"], 2), "peak_tflops": MFMA_F16_PEAK_TFLOPS,
            "frac": round(cm["achieved"] / MFMA_F16_PEAK_TFLOPS, 4),
            "prompt_tokens_per_s": round(cm["prompt_tokens"] / (cm["ms"]["cached"] * 1e-3), 1)}
        result["configs"] = configs
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on bounded samples")
        result["cpu_baseline"] = cpu_baseline(args, w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
