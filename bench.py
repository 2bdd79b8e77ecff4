#!/usr/bin/env python3
"""Benchmark of the paged INT8-KV GQA hot path on one MI355X.

One step = one decode step of a Llama-3.1-8B-shaped attention layer:
kv8_quant_append writes the newest token of each of the 32 sequences into
the INT8 cache, then paged_decode_attn_kv8 attends every sequence's whole
context (1024..4096 tokens, 32 query / 8 KV heads, d = 128).  The cache is
resident in HBM before timing starts; four replicas are rotated so that
the 256 MB last-level cache cannot serve a replica from the previous step.

Prints one JSON line: whole-step algorithmic HBM GB/s as `value`, KV
tokens/s, the decode kernel's roofline fraction (HIP events on the stream
the library launches on), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0     # MI355X dense fp16/bf16 matrix peak
METRIC = "achieved HBM GB/s (% of peak) + KV-tokens/s, paged INT8-KV GQA decode attention"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=3000,
                   help="untimed steps first (the GPU clocks settle over ~100 ms)")
    p.add_argument("--replicas", type=int, default=4)
    p.add_argument("--tokens-per-split", type=int, default=0)
    p.add_argument("--decode-kernel", choices=["auto", "dot", "mfma", "mfma1", "sk"],
                   default="auto",
                   help="form of the INT8/FP8/INT4 decode kernel passed to every decode call "
                        "(auto: the library's choice by group size and size)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-read-ceiling", action="store_true",
                   help="skip the read-only probe that measures the HBM read ceiling")
    p.add_argument("--cpu-steps", type=int, default=24,
                   help="oracle steps timed on the host (about 0.5 s each on 16 cores)")
    p.add_argument("--prefill-steps", type=int, default=20)
    p.add_argument("--fp8-steps", type=int, default=1,
                   help="0 skips the FP8 (e4m3) and INT4 cache lines")
    p.add_argument("--sweep-layers", type=int, default=80,
                   help="layers of the Llama-3-70B-shaped decode sweep (0 skips it)")
    p.add_argument("--fill-steps", type=int, default=20,
                   help="calls of the append fill leg, 131072 tokens each (0 skips it)")
    p.add_argument("--long-steps", type=int, default=64,
                   help="decode steps of the long-context leg, 4 x 32768 tokens (0 skips it)")
    p.add_argument("--long-replicas", type=int, default=3,
                   help="cache copies the long-context leg rotates (each about 273 MB)")
    p.add_argument("--budget-steps", type=int, default=10,
                   help="decode calls timed per side of the 258K equal-budget comparison "
                        "(0 skips it)")
    p.add_argument("--budget-bf16-batch", type=int, default=8,
                   help="sequences the 16-bit cache holds; sets the memory budget")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain elementwise copy of known size (for HBM counters)")
    p.add_argument("--decode-scaling", action="store_true",
                   help="only time the decode against bytes: the Llama-3.1-8B-shaped batch with "
                        "contexts scaled x0.5..x4, every matrix-core form and the random-tile "
                        "read probe on the same bytes (one JSON line)")
    return p.parse_args()


def decode_bytes(ctx, hkv, d, hq, q_bytes):
    """Algorithmic bytes of one decode call: K and V codes plus their fp16
    scales for every attended token and KV head, q, out, block-table entries
    and context lengths."""
    ctx = np.asarray(ctx, np.int64)
    b = len(ctx)
    kv = int(ctx.sum()) * 2 * hkv * (d + 2)
    table = 4 * int(np.sum((ctx + 15) // 16))
    return kv + b * hq * d * q_bytes + b * hq * d * 4 + table + 4 * b


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` ('decode' or 'prefill') from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when the
    kernel's sources changed since those counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        info = json.load(open(os.path.join(root, "profiles", "hbm_traffic.json")))[kernel]
        h = hashlib.sha256()
        for f in info["sources"]:
            h.update(open(os.path.join(root, f), "rb").read())
        if h.hexdigest()[:16] != info["sources_sha256_16"]:
            return None
        return int(info["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def prefill_flops(ctx, chunk, hq, d):
    """Causal-aware FLOPs of one chunked-prefill call: row i of a chunk of
    Lc rows sees ctx - Lc + i + 1 keys; QK^T and PV each cost 2*d per
    (row, head, visible key)."""
    total = 0
    for c, lc in zip(np.asarray(ctx, np.int64), np.asarray(chunk, np.int64)):
        vis = np.arange(c - lc, c) + 1
        total += int(np.clip(vis, 0, None).sum())
    return total * hq * d * 4


def append_bytes(n, hkv, d):
    """Read bf16 K and V, write codes and scales, read slot indices."""
    return n * hkv * d * 2 * 2 + n * hkv * (d + 2) * 2 + 4 * n


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build runs on one GPU; the decode path would shard by sequence or by "
              "KV head, with no exchange inside attention)", file=sys.stderr)
        sys.exit(2)
    import torch
    from paged_int8_kv_amd import binding as B
    from paged_int8_kv_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    args.form = {"auto": B.DECODE_AUTO, "dot": B.DECODE_DOT, "mfma": B.DECODE_MFMA,
                 "mfma1": B.DECODE_MFMA_ONEPASS, "sk": B.DECODE_STREAMK}[args.decode_kernel]
    if args.calibrate_copy:
        calibrate_copy(dev)
        return
    if args.decode_scaling:
        decode_scaling(dev)
        return
    case = W.llama8b_decode()
    bsz, hq, hkv, d = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    ctx = case.context_lens
    max_ctx = int(ctx.max())

    # newest token of every sequence: appended each step
    last = np.cumsum(ctx) - 1
    k_all = torch.from_numpy(case.k_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    v_all = torch.from_numpy(case.v_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    slots_all = torch.from_numpy(case.slot_mapping).to(dev)
    last_t = torch.from_numpy(last).to(dev)
    k_new = k_all.index_select(0, last_t).contiguous()
    v_new = v_all.index_select(0, last_t).contiguous()
    slots_new = slots_all.index_select(0, last_t).contiguous()

    caches = []
    for _ in range(args.replicas):
        c = B.alloc_cache(case.num_blocks, hkv, d, dev)
        B.kv8_quant_append(k_all, v_all, slots_all, *c)
        caches.append(c)
    del k_all, v_all
    q = torch.from_numpy(case.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    table = torch.from_numpy(case.block_table).to(dev)
    lens = torch.from_numpy(ctx).to(dev)
    out = torch.empty((bsz, hq, d), dtype=torch.float32, device=dev)
    ws = torch.zeros(B.kv8_decode_workspace_size(bsz, hq, hkv, d, max_ctx, args.tokens_per_split),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i):
        # one decode step in one launch: append the newest token of every
        # sequence (quantised inside the decode kernel), then attend
        c = caches[i % len(caches)]
        B.paged_decode_attn_kv8_append(q, k_new, v_new, *c, table, lens, max_ctx, out, ws,
                                       tokens_per_split=args.tokens_per_split,
                                       kernel_form=args.form)

    def two_launch_step(i, ev=None):
        c = caches[i % len(caches)]
        if ev is not None:
            ev[0].record()
        B.kv8_quant_append(k_new, v_new, slots_new, *c)
        if ev is not None:
            ev[1].record()
        B.paged_decode_attn_kv8(q, *c, table, lens, max_ctx, out, ws,
                                tokens_per_split=args.tokens_per_split,
                                kernel_form=args.form)
        if ev is not None:
            ev[2].record()

    def timed_steps(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record()
        for i in range(args.steps):
            fn(i)
        t_end.record()
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end)

    # the timed region: exactly K steps, nothing else on the stream
    total_ms = timed_steps(step)
    two_launch_ms = timed_steps(two_launch_step)

    # per-kernel breakdown in a separate pass: events around each launch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        two_launch_step(i, evs[i])
    torch.cuda.synchronize()
    app_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])

    # decode launches back to back (rotating the replicas) between one pair of
    # events: the kernel's own average duration, for the roofline
    n_b2b = max(args.steps, 50)
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    b0.record()
    for i in range(n_b2b):
        c = caches[i % len(caches)]
        B.paged_decode_attn_kv8(q, *c, table, lens, max_ctx, out, ws,
                                tokens_per_split=args.tokens_per_split,
                                kernel_form=args.form)
    b1.record()
    torch.cuda.synchronize()
    dec_b2b_us = b0.elapsed_time(b1) / n_b2b * 1e3

    # the append alone, back to back: plain, and with RoPE fused in front of
    # the quantiser (positions of the newest tokens, Llama-3 table)
    table = torch.from_numpy(W.rope_cos_sin(8192, d)).to(dev)
    pos_new = torch.from_numpy((ctx - 1).astype(np.int32)).to(dev)

    def b2b(fn, n=50):
        for _ in range(5):
            fn(0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    app_plain_us = b2b(lambda i: B.kv8_quant_append(k_new, v_new, slots_new,
                                                    *caches[i % len(caches)]))
    app_rope_us = b2b(lambda i: B.kv8_rope_quant_append(k_new, v_new, slots_new, pos_new, table,
                                                        *caches[i % len(caches)]))

    step_ms = total_ms / args.steps
    d_bytes = decode_bytes(ctx, hkv, d, hq, 2)
    a_bytes = append_bytes(bsz, hkv, d)
    step_gbs = (d_bytes + a_bytes) / (step_ms * 1e-3) / 1e9
    dec_avg = float(dec_ms.mean())
    dec_gbs = d_bytes / (dec_b2b_us * 1e-6) / 1e9
    kv_tok_s = float(ctx.sum()) / (step_ms * 1e-3)

    result = {
        "metric": METRIC,
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 operands (int8 codes exact in f16, q rescaled by a power of two, "
                 "weights p*v_scale), f32 accumulation and softmax",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3.1-8B-shaped decode layer: append 1 token/seq + paged INT8-KV "
                        "GQA decode in one launch (paged_decode_attn_kv8_append); B=32, Hq=32, "
                        "Hkv=8, d=128, ctx~U[1024,4096], block 16",
            "kv_dtype": "int8 codes + fp16 per-token scales",
            "q_dtype": "bf16",
            "sum_ctx": int(ctx.sum()),
            "replicas_rotated": len(caches),
            "tokens_per_split": args.tokens_per_split or "library default",
        },
        "pct_of_hbm_peak": round(100.0 * step_gbs / HBM_PEAK_GBS, 2),
        "kv_tokens_per_s": round(kv_tok_s, 1),
        "decode_us": {"mean": round(dec_avg * 1e3, 2),
                      "p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                      "p50": round(float(np.percentile(dec_ms, 50)) * 1e3, 2),
                      "p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2)},
        "decode_back_to_back_us": round(dec_b2b_us, 2),
        "append_us": {"mean": round(float(app_ms.mean()) * 1e3, 2)},
        "two_launch_step_us": round(two_launch_ms / args.steps * 1e3, 2),
        "append_back_to_back_us": {"plain": round(app_plain_us, 2),
                                   "rope_fused": round(app_rope_us, 2)},
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode"),
                     "kernel": "paged_decode_attn_kv8 (one launch, split-K + in-launch merge); "
                               "duration from back-to-back launches",
                     "bytes_per_launch": d_bytes},
    }
    del caches, ws, out
    torch.cuda.empty_cache()
    if not args.no_read_ceiling:
        tiles = bench_read_ceiling(dev, d_bytes)
        stream = bench_stream_read(dev)
        best = max(tiles["gbs"], stream["gbs"])
        result["read_ceiling"] = {"gbs": best, "pct_of_hbm_peak": round(best / HBM_PEAK_GBS * 100, 2),
                                  "stream": stream, "random_tiles": tiles,
                                  "note": "the larger of the two measured read rates"}
        result["roofline"]["frac_of_read_ceiling"] = round(dec_gbs / best, 4)
    if args.prefill_steps > 0:
        result["prefill"] = bench_prefill(args, dev)
    if args.fp8_steps > 0:
        result["fp8_kv"] = {"decode": bench_code_decode(args, dev, case, "fp8")}
        if args.prefill_steps > 0:
            result["fp8_kv"]["prefill"] = bench_prefill(args, dev, fp8=True)
    if args.fp8_steps > 0:
        result["int4_kv"] = {"decode": bench_code_decode(args, dev, case, "int4")}
        if args.prefill_steps > 0:
            result["int4_kv"]["prefill"] = bench_prefill(args, dev, int4=True)
    if args.fill_steps > 0:
        result["append_fill"] = bench_append_fill(args, dev)
    if args.long_steps > 0:
        result["long_context"] = bench_long_context(args, dev)
    if args.sweep_layers > 0:
        result["llama70b_sweep"] = bench_sweep70b(args, dev)
    if args.budget_steps > 0:
        result["equal_budget_258k"] = bench_equal_budget(args, dev)
    if "read_ceiling" in result:
        ceil = result["read_ceiling"]["gbs"]
        for leg in ("long_context", "llama70b_sweep"):
            if leg in result:
                result[leg]["frac_of_read_ceiling"] = round(result[leg]["kv_gbs"] / ceil, 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_steps, d_bytes + a_bytes)
    print(json.dumps(result), flush=True)


def bench_prefill(args, dev, fp8=False, int4=False):
    """Chunked prefill over the INT8 (or FP8, or INT4) cache (batch 8, 32/8 heads,
    d=128, 2048..8192 earlier tokens + a 512-row causal chunk): per step,
    append the chunk's own K/V (4096 tokens), then the prefill call.  HIP
    events on the stream the library launches on."""
    import torch
    from paged_int8_kv_amd import binding as B
    from paged_int8_kv_amd import workloads as W
    case = W.chunked_prefill()
    hq, hkv, d = case.num_q_heads, case.num_kv_heads, case.head_dim
    chunk = case.extra["chunk"]
    ctx = case.context_lens
    mask = case.extra["chunk_mask"]
    k_all = torch.from_numpy(case.k_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    v_all = torch.from_numpy(case.v_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    fmt = "int4" if int4 else ("fp8" if fp8 else "kv8")
    append = {"int4": B.kv8_quant_append_int4, "fp8": B.kv8_quant_append_fp8,
              "kv8": B.kv8_quant_append}[fmt]
    prefill = {"int4": B.paged_prefill_chunk_attn_int4kv, "fp8": B.paged_prefill_chunk_attn_fp8kv,
               "kv8": B.paged_prefill_chunk_attn_kv8}[fmt]
    cache = B.alloc_cache(case.num_blocks, hkv, d, dev, fp8=fp8, int4=int4)
    append(k_all, v_all, torch.from_numpy(case.slot_mapping).to(dev), *cache)
    sel = torch.from_numpy(np.nonzero(mask)[0]).to(dev)
    k_new = k_all.index_select(0, sel).contiguous()
    v_new = v_all.index_select(0, sel).contiguous()
    s_new = torch.from_numpy(case.slot_mapping[mask]).to(dev)
    del k_all, v_all
    q = torch.from_numpy(case.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    qsl = torch.from_numpy(case.extra["q_start_loc"]).to(dev)
    table = torch.from_numpy(case.block_table).to(dev)
    lens = torch.from_numpy(ctx).to(dev)
    out = torch.empty((q.shape[0], hq, d), dtype=torch.float32, device=dev)
    max_ctx = int(ctx.max())

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        append(k_new, v_new, s_new, *cache)
        if ev is not None:
            ev[1].record()
        prefill(q, qsl, chunk, *cache, table, lens, max_ctx, out)
        if ev is not None:
            ev[2].record()

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(args.prefill_steps)]
    for i in range(args.prefill_steps):
        step(evs[i])
    torch.cuda.synchronize()
    app = np.array([e[0].elapsed_time(e[1]) for e in evs])
    pre = np.array([e[1].elapsed_time(e[2]) for e in evs])
    flops = prefill_flops(ctx, np.full(len(ctx), chunk), hq, d)
    tf = flops / (float(pre.mean()) * 1e-3) / 1e12
    return {"workload": "chunked prefill: B=8, Hq=32, Hkv=8, d=128, ctx_prev~U[2048,8192] + "
                        f"512-row causal chunk, bf16 Q, "
                        f"{ {'int4': 'int4', 'fp8': 'fp8 e4m3', 'kv8': 'int8'}[fmt]} KV cache",
            "steps": args.prefill_steps,
            "prefill_us": {"mean": round(float(pre.mean()) * 1e3, 2),
                           "p50": round(float(np.percentile(pre, 50)) * 1e3, 2)},
            "append_chunk_us": {"mean": round(float(app.mean()) * 1e3, 2)},
            "flops_per_call": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill") if fmt == "kv8" else None,
                         "kernel": prefill.__name__ + " (fp16 MFMA 32x32x16)"}}


def bench_code_decode(args, dev, case, fmt):
    """Decode over an FP8 (e4m3) or INT4 cache on the same decode workload,
    cache written by the matching append, launches back to back over
    rotated replicas.  Algorithmic bytes as for INT8 with the code bytes of
    the format (d for FP8, d/2 for INT4)."""
    import torch
    from paged_int8_kv_amd import binding as B
    bsz, hq, hkv, d = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    ctx = case.context_lens
    max_ctx = int(ctx.max())
    int4 = fmt == "int4"
    append = B.kv8_quant_append_int4 if int4 else B.kv8_quant_append_fp8
    decode = B.paged_decode_attn_int4kv if int4 else B.paged_decode_attn_fp8kv
    k_all = torch.from_numpy(case.k_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    v_all = torch.from_numpy(case.v_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    caches = []
    for _ in range(args.replicas):
        c = B.alloc_cache(case.num_blocks, hkv, d, dev, fp8=not int4, int4=int4)
        append(k_all, v_all, slots, *c)
        caches.append(c)
    del k_all, v_all
    q = torch.from_numpy(case.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    table = torch.from_numpy(case.block_table).to(dev)
    lens = torch.from_numpy(ctx).to(dev)
    out = torch.empty((bsz, hq, d), dtype=torch.float32, device=dev)
    ws = torch.zeros(B.kv8_decode_workspace_size(bsz, hq, hkv, d, max_ctx, args.tokens_per_split),
                     dtype=torch.uint8, device=dev)
    n = max(args.steps, 50)
    for i in range(200):
        decode(q, *caches[i % len(caches)], table, lens, max_ctx, out, ws,
               tokens_per_split=args.tokens_per_split,
               kernel_form=args.form)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        decode(q, *caches[i % len(caches)], table, lens, max_ctx, out, ws,
               tokens_per_split=args.tokens_per_split,
               kernel_form=args.form)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    code_bytes = d // 2 if int4 else d
    nbytes = (int(ctx.sum()) * 2 * hkv * (code_bytes + 2) + bsz * hq * d * 2 + bsz * hq * d * 4
              + 4 * int(np.sum((ctx + 15) // 16)) + 4 * bsz)
    del caches, ws, out
    torch.cuda.empty_cache()
    return {"workload": f"the decode layer above over an {'INT4' if int4 else 'FP8 (e4m3)'} "
                        "cache, decode launches back to back", "decode_us": round(us, 2),
            "bytes_per_launch": nbytes, "kv_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "kv_tokens_per_s": round(float(ctx.sum()) / (us * 1e-6), 1)}


def bench_append_fill(args, dev, n_tokens=131072, hkv=8, d=128):
    """kv8_quant_append at fill size: 131072 new tokens (4 sequences of
    32768, the long-context config's fill), 8 KV heads, d=128, bf16 K/V
    drawn on the device, slots a random permutation of the cache (numpy
    PCG64 seeded 13); calls back to back between HIP events."""
    import torch
    from paged_int8_kv_amd import binding as B
    nb = n_tokens // 16
    gen = torch.Generator(device=dev)
    gen.manual_seed(13)
    k = torch.randn((n_tokens, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn((n_tokens, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    rng = np.random.Generator(np.random.PCG64(13))
    blocks = rng.permutation(nb).astype(np.int64)
    slots_np = (blocks[:, None] * 16 + np.arange(16)[None, :]).reshape(-1).astype(np.int32)
    slots = torch.from_numpy(slots_np).to(dev)
    cache = B.alloc_cache(nb, hkv, d, dev)
    for _ in range(3):
        B.kv8_quant_append(k, v, slots, *cache)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.fill_steps):
        B.kv8_quant_append(k, v, slots, *cache)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.fill_steps
    nbytes = append_bytes(n_tokens, hkv, d)
    del k, v, slots, cache
    torch.cuda.empty_cache()
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"kv8_quant_append fill: {n_tokens} tokens, Hkv={hkv}, d={d}, bf16 K/V, "
                        "random block order, calls back to back",
            "us_per_call": round(us, 2), "bytes_per_call": int(nbytes),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "tokens_per_s": round(n_tokens / (us * 1e-6), 1)}


def probe_workgroups(dev, per_cu=4):
    """Persistent workgroups of the read-ceiling kernels: a few per CU."""
    import torch
    return per_cu * torch.cuda.get_device_properties(dev).multi_processor_count


def bench_read_ceiling(dev, n_bytes, tile_bytes=2048, buffer_bytes=1 << 30, replicas=4,
                       launches=100):
    """The measured HBM read rate of the decode's access pattern: the
    library's kv8_read_probe streams about n_bytes per launch as random
    tile_bytes tiles (one (block, KV head) code tile of the decode) out of a
    1 GiB buffer, rotating `replicas` tile orders, each wave of the
    persistent workgroups streaming its own tiles, launches back to back
    between HIP events on the current stream."""
    import torch
    from paged_int8_kv_amd import binding as B
    n_tiles_read = max(1, n_bytes // tile_bytes)
    n_read = n_tiles_read * tile_bytes
    n_tiles_buf = buffer_bytes // tile_bytes
    buf = torch.zeros(buffer_bytes, dtype=torch.uint8, device=dev)
    rng = np.random.Generator(np.random.PCG64(11))
    orders = [torch.from_numpy(rng.permutation(n_tiles_buf)[:n_tiles_read].astype(np.int32)).to(dev)
              for _ in range(replicas)]
    wg = probe_workgroups(dev)
    out = torch.empty(wg * 256, dtype=torch.int32, device=dev)
    for i in range(20):
        B.kv8_read_probe(buf, orders[i % replicas], tile_bytes, wg, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(launches):
        B.kv8_read_probe(buf, orders[i % replicas], tile_bytes, wg, out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    del buf, orders, out
    torch.cuda.empty_cache()
    return {"kernel": "kv8_read_probe: read-only, random tiles streamed per wave, "
                      "persistent workgroups, ordinary 16-byte loads, 4 KB in flight per wave",
            "tile_bytes": tile_bytes, "buffer_bytes": buffer_bytes, "bytes_per_launch": int(n_read),
            "workgroups": wg, "us_per_launch": round(us, 2),
            "gbs": round(n_read / (us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(n_read / (us * 1e-6) / 1e9 / HBM_PEAK_GBS * 100, 2)}


def bench_stream_read(dev, buffer_bytes=2 << 30, launches=30):
    """The plain streaming read rate of HBM: the library's kv8_stream_read
    over a 2 GiB buffer (eight times the last-level cache), persistent
    workgroups with nontemporal loads, launches back to back between HIP
    events on the current stream."""
    import torch
    from paged_int8_kv_amd import binding as B
    chunk = B.load().kv8_read_probe_chunk_bytes()
    buf = torch.zeros(buffer_bytes // chunk * chunk, dtype=torch.uint8, device=dev)
    wg = probe_workgroups(dev)
    out = torch.empty(wg * 256, dtype=torch.int32, device=dev)
    for _ in range(5):
        B.kv8_stream_read(buf, wg, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        read = B.kv8_stream_read(buf, wg, out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    del buf, out
    torch.cuda.empty_cache()
    return {"kernel": "kv8_stream_read: read-only, contiguous, persistent workgroups, "
                      "nontemporal 16-byte loads",
            "buffer_bytes": int(read), "workgroups": wg, "us_per_launch": round(us, 2),
            "gbs": round(read / (us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(read / (us * 1e-6) / 1e9 / HBM_PEAK_GBS * 100, 2)}


def bench_long_context(args, dev, batch=4, ctx0=32768):
    """Long-context decode with append: 4 sequences of 32768 tokens, 32/8
    heads, d=128, fp32 q; each step appends one token per sequence and
    decodes over the grown context in one launch
    (paged_decode_attn_kv8_append), `long_steps` steps back to back.  K/V/q
    are drawn N(0, 1) on the device (torch.Generator seeded 3000), the
    context quantised by the append kernel; the block table is a random
    permutation (numpy PCG64 seeded 3) with room for every step.

    One cache is about 273 MB, close to the 256 MB last-level cache, so
    `long_replicas` copies of the cache are rotated step by step (3 by
    default: 820 MB between two reads of one copy).  Every copy is filled
    beforehand with the same tokens, those the steps append included, so a
    step's append rewrites the values its copy already holds and every copy
    holds the whole sequence whichever step reads it."""
    import torch
    from paged_int8_kv_amd import binding as B
    steps, hq, hkv, d = args.long_steps, 32, 8, 128
    reps = max(1, args.long_replicas)
    ctx_max = ctx0 + steps
    bps = -(-ctx_max // 16)
    nb = batch * bps
    rng = np.random.Generator(np.random.PCG64(3))
    table_np = rng.permutation(nb).astype(np.int32).reshape(batch, bps)
    pos = np.arange(ctx0)
    slots_np = np.concatenate([table_np[b][pos // 16] * 16 + pos % 16 for b in range(batch)])
    gen = torch.Generator(device=dev)
    gen.manual_seed(3000)
    caches = [B.alloc_cache(nb, hkv, d, dev) for _ in range(reps)]
    for b in range(batch):      # one sequence at a time keeps the bf16 staging small
        k = torch.randn((ctx0, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((ctx0, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
        sl = torch.from_numpy(np.ascontiguousarray(slots_np[b * ctx0:(b + 1) * ctx0])).to(dev)
        for c in caches:
            B.kv8_quant_append(k, v, sl, *c)
        del k, v
    k_new = torch.randn((steps, batch, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    v_new = torch.randn((steps, batch, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    q = torch.randn((steps, batch, hq, d), generator=gen, device=dev)
    lens_np = ctx0 + 1 + np.arange(steps, dtype=np.int32)[:, None].repeat(batch, 1)
    for st in range(steps):     # the appended tokens, into every copy beforehand
        p = ctx0 + st
        sl = torch.from_numpy((table_np[:, p // 16] * 16 + p % 16).astype(np.int32)).to(dev)
        for c in caches:
            B.kv8_quant_append(k_new[st], v_new[st], sl, *c)
    lens = torch.from_numpy(np.ascontiguousarray(lens_np)).to(dev)
    table = torch.from_numpy(table_np).to(dev)
    ws = torch.zeros(B.kv8_decode_workspace_size(batch, hq, hkv, d, ctx_max, args.tokens_per_split),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((batch, hq, d), dtype=torch.float32, device=dev)

    def run():
        for s in range(steps):
            B.paged_decode_attn_kv8_append(q[s], k_new[s], v_new[s], *caches[s % reps], table,
                                           lens[s], ctx_max, out, ws,
                                           tokens_per_split=args.tokens_per_split,
                                           kernel_form=args.form)

    run()
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    us = float(np.median(times)) * 1e3 / steps
    nbytes = float(np.mean([decode_bytes(lens_np[s], hkv, d, hq, 4) for s in range(steps)]))
    nbytes += append_bytes(batch, hkv, d)
    tokens = float(lens_np.sum()) / steps
    del caches, k_new, v_new, q, ws, out
    torch.cuda.empty_cache()
    return {"workload": f"long-context decode with append: B={batch}, Hq={hq}, Hkv={hkv}, d={d}, "
                        f"ctx {ctx0} + 1 token per sequence per step, fp32 q, {steps} steps "
                        f"back to back (paged_decode_attn_kv8_append), {reps} cache copies "
                        "rotated step by step",
            "replicas_rotated": reps,
            "us_per_step": round(us, 2), "bytes_per_step": int(nbytes),
            "kv_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / 8000 * 100, 2),
            "kv_tokens_per_s": round(tokens / (us * 1e-6), 1)}


def bench_sweep70b(args, dev):
    """The Llama-3-70B-shaped decode sweep: one decode call per layer, all
    layers back to back as one model step launches them (64 sequences of
    512..16384 tokens per layer, 64 query heads over 8 KV heads, d=128,
    K/V drawn on the device and quantised by the append kernel; about 49 GB
    of cache for 80 layers, far beyond the last-level cache)."""
    import torch
    from paged_int8_kv_amd import binding as B
    from paged_int8_kv_amd import workloads as W
    layers = []
    kv_bytes = 0
    tokens = 0
    for layer in range(args.sweep_layers):
        g = W.llama70b_layer_device(layer, dev)
        cache = B.alloc_cache(g["num_blocks"], 8, 128, dev)
        B.kv8_quant_append(g["k"], g["v"], torch.from_numpy(g["slot_mapping"]).to(dev), *cache)
        lens = g["context_lens"]
        layers.append((g["q"], cache, torch.from_numpy(g["block_table"]).to(dev),
                       torch.from_numpy(lens).to(dev), int(lens.max())))
        kv_bytes += decode_bytes(lens, 8, 128, 64, 2)
        tokens += int(lens.astype(np.int64).sum())
        del g
    torch.cuda.synchronize()
    max_ctx = max(x[4] for x in layers)
    ws = torch.zeros(B.kv8_decode_workspace_size(64, 64, 8, 128, max_ctx, args.tokens_per_split),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((64, 64, 128), dtype=torch.float32, device=dev)

    def sweep():
        for q, cache, table, lens, m in layers:
            B.paged_decode_attn_kv8(q, *cache, table, lens, m, out, ws,
                                    tokens_per_split=args.tokens_per_split,
                                    kernel_form=args.form)

    for _ in range(3):
        sweep()
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        sweep()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    del layers, ws, out
    torch.cuda.empty_cache()
    return {"workload": f"Llama-3-70B-shaped decode sweep: {args.sweep_layers} layers back to "
                        "back, B=64, Hq=64, Hkv=8, d=128, ctx ~ log-U[512,16384] per layer",
            "ms_per_step": round(ms, 3),
            "us_per_layer": round(ms * 1e3 / args.sweep_layers, 1),
            "bytes_per_step": int(kv_bytes), "kv_gbs": round(gbs, 1),
            "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
            "kv_tokens_per_s": round(tokens / (ms * 1e-3), 1)}


def bench_equal_budget(args, dev):
    """Decode at 258K tokens per sequence with one per-layer KV memory
    budget for both caches: the budget holds budget_bf16_batch sequences of
    bf16 K/V, and as many INT8 sequences (codes + fp16 scales) as fit in the
    same bytes.  Both sides hold the same seeded tokens and queries for the
    sequences they share.  Reports decode tokens/s (sequences / call time)
    for each side and their ratio, the comparison the KV8 README draws
    against FlashAttention-2 at 258K context (1.64x on its own system)."""
    import torch
    from paged_int8_kv_amd import binding as B
    from paged_int8_kv_amd import workloads as W
    hq, hkv, d = 32, 8, 128
    ctx = 258 * 1024
    per_tok_bf16 = 2 * hkv * d * 2
    per_tok_int8 = 2 * hkv * (d + 2)
    b16 = args.budget_bf16_batch
    budget = b16 * ctx * per_tok_bf16
    b8 = budget // (ctx * per_tok_int8)

    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3     # us per call

    per_tok_int4 = 2 * hkv * (d // 2 + 2)
    b4 = budget // (ctx * per_tok_int4)
    res = {"workload": f"decode, Llama-3.1-8B attention (Hq=32, Hkv=8, d=128), {ctx} tokens per "
                       "sequence, bf16 q, one KV budget per layer",
           "context_tokens": ctx, "budget_bytes": int(budget),
           "bf16_kv": {"batch": b16}, "int8_kv": {"batch": int(b8)}, "int4_kv": {"batch": int(b4)}}
    outs = {}
    for kind, batch in (("bf16_kv", b16), ("int8_kv", int(b8)), ("int4_kv", int(b4))):
        w = W.long_context_258k(batch, dev)
        nb = w["num_blocks"]
        table = torch.from_numpy(w["block_table"]).to(dev)
        lens = torch.from_numpy(w["context_lens"]).to(dev)
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=dev)
        ws = torch.zeros(B.kv8_decode_workspace_size(batch, hq, hkv, d, ctx, 0),
                         dtype=torch.uint8, device=dev)
        if kind == "bf16_kv":
            kc = torch.empty((nb, hkv, 16, d), dtype=torch.bfloat16, device=dev)
            vc = torch.empty_like(kc)
            for b in range(batch):
                k, v = w["tokens"](b)
                s = w["slots"](b).long()
                kc[s // 16, :, s % 16, :] = k
                vc[s // 16, :, s % 16, :] = v
                del k, v, s
            cache = (kc, vc)
            call = lambda: B.paged_decode_attn_bf16kv(w["q"], *cache, table, lens, ctx, out, ws)
            nbytes = batch * ctx * per_tok_bf16
        elif kind == "int8_kv":
            cache = B.alloc_cache(nb, hkv, d, dev)
            for b in range(batch):
                k, v = w["tokens"](b)
                B.kv8_quant_append(k, v, w["slots"](b), *cache)
                del k, v
            call = lambda: B.paged_decode_attn_kv8(w["q"], *cache, table, lens, ctx, out, ws,
                                                   kernel_form=args.form)
            nbytes = batch * ctx * per_tok_int8
        else:
            cache = B.alloc_cache(nb, hkv, d, dev, int4=True)
            for b in range(batch):
                k, v = w["tokens"](b)
                B.kv8_quant_append_int4(k, v, w["slots"](b), *cache)
                del k, v
            call = lambda: B.paged_decode_attn_int4kv(w["q"], *cache, table, lens, ctx, out, ws,
                                                      kernel_form=args.form)
            nbytes = batch * ctx * per_tok_int4
        torch.cuda.synchronize()
        us = timed(call, args.budget_steps)
        outs[kind] = out.clone()
        res[kind].update({"decode_us": round(us, 1),
                          "decode_tokens_per_s": round(batch / (us * 1e-6), 1),
                          "kv_tokens_per_s": round(batch * ctx / (us * 1e-6), 1),
                          "kv_gbs": round(nbytes / (us * 1e-6) / 1e9, 1)})
        del cache, ws, out, table, lens, w
        torch.cuda.empty_cache()
    res["throughput_ratio_int8_over_bf16"] = round(
        res["int8_kv"]["decode_tokens_per_s"] / res["bf16_kv"]["decode_tokens_per_s"], 3)
    res["throughput_ratio_int4_over_bf16"] = round(
        res["int4_kv"]["decode_tokens_per_s"] / res["bf16_kv"]["decode_tokens_per_s"], 3)
    n = min(b16, int(b8))
    res["int8_vs_bf16_output_max_abs"] = float(
        (outs["int8_kv"][:n] - outs["bf16_kv"][:n]).abs().max().item())
    res["int4_vs_bf16_output_max_abs"] = float(
        (outs["int4_kv"][:n] - outs["bf16_kv"][:n]).abs().max().item())
    res["pages_figure"] = "1.64x KV8 over FA2 at 258K, same memory budget, L40S, system level"
    return res


def decode_scaling(dev, scales=(0.5, 1.0, 2.0, 4.0), launches=100, seed=12):
    """Decode time against bytes.  The Llama-3.1-8B-shaped batch (32
    sequences, 32/8 heads, d=128, bf16 q) with contexts U[1024 f, 4096 f]
    for each f: random codes and scales drawn on the device (the kernels'
    time does not depend on the values), a permuted block table, enough
    cache copies rotated back to back to pass the last-level cache.  Each
    matrix-core form, and the random-tile read probe over the same bytes.
    The line through the two smallest points gives each form's fixed cost
    (intercept) and streaming rate (slope) where its grid is one round; the
    line through the two largest, the same at sizes of several rounds."""
    import torch
    from paged_int8_kv_amd import binding as B
    hq, hkv, d, bsz = 32, 8, 128, 32
    forms = {"two_pass": B.DECODE_MFMA, "one_pass": B.DECODE_MFMA_ONEPASS,
             "stream_k": B.DECODE_STREAMK}
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    rows = []
    for f in scales:
        rng = np.random.Generator(np.random.PCG64(seed))
        ctx = rng.integers(int(1024 * f), int(4096 * f) + 1, size=bsz)
        nb = (ctx + 15) // 16
        nblocks, maxb = int(nb.sum()), int(nb.max())
        perm = rng.permutation(nblocks).astype(np.int32)
        table = np.zeros((bsz, maxb), np.int32)
        o = 0
        for b in range(bsz):
            table[b, :nb[b]] = perm[o:o + nb[b]]
            o += nb[b]
        nbytes = decode_bytes(ctx, hkv, d, hq, 2)
        reps = max(2, int(np.ceil(800e6 / nbytes)))
        caches = []
        for _ in range(reps):
            kc, vc, ks, vs = B.alloc_cache(nblocks, hkv, d, dev)
            kc.copy_(torch.randint(-127, 128, kc.shape, dtype=torch.int8, device=dev, generator=gen))
            vc.copy_(torch.randint(-127, 128, vc.shape, dtype=torch.int8, device=dev, generator=gen))
            for sc in (ks, vs):
                sc.copy_((torch.rand(sc.shape, device=dev, generator=gen) * 0.05 + 0.01)
                         .half().view(torch.int16))
            caches.append((kc, vc, ks, vs))
        q = torch.randn((bsz, hq, d), device=dev, generator=gen).to(torch.bfloat16)
        tab = torch.from_numpy(table).to(dev)
        lens = torch.from_numpy(ctx.astype(np.int32)).to(dev)
        out = torch.empty((bsz, hq, d), dtype=torch.float32, device=dev)
        ws = torch.zeros(B.kv8_decode_workspace_size(bsz, hq, hkv, d, int(ctx.max()), 0),
                         dtype=torch.uint8, device=dev)
        row = {"scale": f, "bytes_per_call": int(nbytes), "us": {}}
        for name, form in forms.items():
            def call(i):
                B.paged_decode_attn_kv8(q, *caches[i % reps], tab, lens, int(ctx.max()), out, ws,
                                        kernel_form=form)
            for i in range(30):
                call(i)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(launches):
                call(i)
            e1.record()
            torch.cuda.synchronize()
            row["us"][name] = round(e0.elapsed_time(e1) * 1e3 / launches, 2)
        del caches, ws
        torch.cuda.empty_cache()
        row["us"]["read_probe"] = bench_read_ceiling(dev, nbytes)["us_per_launch"]
        rows.append(row)
        print(f"scale {f}: {row}", file=sys.stderr, flush=True)
    def line(r0, r1, name):
        x0, x1 = r0["bytes_per_call"], r1["bytes_per_call"]
        y0, y1 = r0["us"][name], r1["us"][name]
        slope = (y1 - y0) / (x1 - x0)                   # us per byte
        return {"fixed_us": round(y0 - slope * x0, 2), "stream_gbs": round(1e-3 / slope, 1)}
    fits = {name: {"smallest_two": line(rows[0], rows[1], name),
                   "largest_two": line(rows[-2], rows[-1], name)}
            for name in list(forms) + ["read_probe"]}
    print(json.dumps({"decode_scaling": "Llama-3.1-8B-shaped batch, contexts U[1024 f, 4096 f]",
                      "points": rows, "lines": fits}), flush=True)


def calibrate_copy(dev, n_bytes=256 << 20, launches=5):
    """A plain elementwise kernel that reads n_bytes and writes n_bytes per
    launch: the reference against which the HBM byte counters (FETCH_SIZE,
    WRITE_SIZE) of the attention kernels are scaled."""
    import torch
    x = torch.ones(n_bytes // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(launches):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise copy y = x * 1.0 (fp32)",
                      "bytes_read_per_launch": n_bytes, "bytes_written_per_launch": n_bytes,
                      "launches": launches}), flush=True)


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, n_steps, step_bytes):
    """The fp64 oracle on the host: the same step (append the newest token of
    every sequence, then decode the whole batch), repeated n_steps times."""
    from oracle import kv8_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    kc, vc, ks, vs = O.alloc_paged_cache(case.num_blocks, case.num_kv_heads, case.head_dim)
    O.quant_append(case.k, case.v, case.slot_mapping, kc, vc, ks, vs)
    last = np.cumsum(case.context_lens) - 1
    t0 = time.perf_counter()
    for _ in range(n_steps):
        O.quant_append(case.k[last], case.v[last], case.slot_mapping[last], kc, vc, ks, vs)
        O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    dt = (time.perf_counter() - t0) / n_steps
    return {"value": round(step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "cpu_model": cpu_model(), "host_cpus_usable": len(os.sched_getaffinity(0)),
            "kind": "oracle", "seconds_per_step": round(dt, 3),
            "kv_tokens_per_s": round(float(case.context_lens.sum()) / dt, 1),
            "sample": f"{n_steps} full steps of the same workload (append 32 tokens + decode "
                      f"all 32 sequences), numpy fp64 oracle"}


if __name__ == "__main__":
    main()
