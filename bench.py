#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV cache on one MI355X.

One step = the decode step's device work on inputs resident in HBM:
  reshape_and_cache (write each sequence's new token into its slot)
  + paged_attention_decode (one query token per sequence over its paged context)
on the 13B-shaped workload (40 heads x 128, fp16, block 16, 30 sequences, context U[128, 2048]).
Slot assignment for the step is done once by the host allocator before timing.

Prints ONE JSON line. KV GB/s counts algorithmic bytes (each context token's K and V rows once,
q in, out, table entries, lengths; plus the new tokens' K/V read and written).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV GB/s (% HBM peak) and decode tokens/s, 13B shape"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s


def attention_bytes(ctx, hq, hkv, d, elt, bs):
    """Algorithmic bytes of one decode-attention call."""
    kv = sum(int(c) for c in ctx) * 2 * hkv * d * elt
    qo = 2 * len(ctx) * hq * d * elt
    tables = sum(-(-int(c) // bs) for c in ctx) * 4
    return kv + qo + tables + 4 * len(ctx)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="13b", choices=["13b", "sweep-b8", "sweep-b16", "sweep-b32", "gqa"])
    ap.add_argument("--partition", type=int, default=-1, help="partition size; -1 = the workload's default")
    ap.add_argument("--replicas", type=int, default=3, help="cache copies rotated across steps (defeats the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-contiguous", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after timing, run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def make_workload(name):
    import synth
    if name == "13b":
        return synth.llama13b(), 0
    if name.startswith("sweep-b"):
        return synth.block_sweep(block_size=int(name[7:])), 0
    if name == "gqa":
        return synth.gqa_shared_prefix(), 512
    raise ValueError(name)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the path shards by sequence "
              f"or KV head with no exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_416_amd import kernels
    from paged_kv_cache_416_amd.cache import PagedKVCache, run_ops, to_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w, default_P = make_workload(args.workload)
    P = default_P if args.partition < 0 else args.partition
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    S, hq, hkv, d, B, elt = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.elt_bytes

    # build the cache state: every op but the decode step's own append
    cache = PagedKVCache(w.num_blocks, B, hkv, d, dt, device=dev, free_order=w.free_order)
    run_ops(cache, w.ops[:-1], dt)
    step = w.ops[-1][1]  # [(sid, k[1,Hkv,D], v[1,Hkv,D]), ...]
    slots, pairs = cache.pool.append([(sid, k.shape[0]) for sid, k, _ in step])
    assert len(pairs) == 0
    new_k = to_device(np.concatenate([k for _, k, _ in step]), dt, dev)
    new_v = to_device(np.concatenate([v for _, _, v in step]), dt, dev)
    slot_dev = torch.from_numpy(slots).to(dev)
    tb, ctx_dev, max_ctx = cache.tables(w.batch)
    ctx = w.final_lengths()
    q = to_device(w.q, dt, dev)
    out = torch.empty_like(q)
    ws = kernels.alloc_workspace(S, hq, d, max_ctx, P, dev)
    ks = [cache.k] + [cache.k.clone() for _ in range(args.replicas - 1)]
    vs = [cache.v] + [cache.v.clone() for _ in range(args.replicas - 1)]
    torch.cuda.synchronize()

    a_bytes = attention_bytes(ctx, hq, hkv, d, elt, B)
    w_bytes = 2 * 2 * len(step) * hkv * d * elt + 8 * len(step)  # K1: read + write K and V, slots
    stream = torch.cuda.current_stream()

    def one_step(i, ev=None):
        r = i % args.replicas
        kernels.reshape_and_cache(new_k, new_v, ks[r], vs[r], slot_dev)
        if ev is not None:
            ev[0].record(stream)
        kernels.paged_attention_decode(out, q, ks[r], vs[r], tb, ctx_dev, max_ctx, w.scale, P, ws, args.flags)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    # timed region: whole steps, host clock
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # attention launches alone, HIP events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        one_step(i, evs[i])
    torch.cuda.synchronize()
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    attn_avg_us = 1e3 * sum(attn_ms) / len(attn_ms)
    attn_med_us = 1e3 * sorted(attn_ms)[len(attn_ms) // 2]

    value = (a_bytes + w_bytes) / (ms_per_step * 1e-3) / 1e9
    achieved = a_bytes / (attn_avg_us * 1e-6) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1)*0.5 keys/values, uniform context lengths)",
        "config": {"workload": w.name, "num_seqs": S, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
                   "block_size": B, "sum_context": int(ctx.sum()), "max_context": int(ctx.max()),
                   "partition_size": P, "replicas": args.replicas},
        "pct_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "decode_tokens_per_s": round(S / (ms_per_step * 1e-3), 1),
        "attention_us": {"avg": round(attn_avg_us, 2), "median": round(attn_med_us, 2)},
        "bytes_per_step": {"attention": a_bytes, "cache_write": w_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "attn_decode_kernel" + ("+attn_reduce_kernel" if P else "")},
    }

    if args.copy_probe:
        src = torch.empty(args.copy_probe << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
        del src, dst

    if not args.no_contiguous:
        result["contiguous"] = contiguous_leg(w, P, args, dev, dt, attn_avg_us)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, P, a_bytes, args.cpu_seconds)

    print(json.dumps(result), flush=True)


def contiguous_leg(w, P, args, dev, dt, paged_us):
    """The same attention on a contiguous [S, Hkv, Lmax, D] cache: the indirection's price."""
    import numpy as np
    import torch

    import synth
    from paged_kv_cache_416_amd import kernels
    from paged_kv_cache_416_amd.cache import to_device

    ctx = w.final_lengths()
    lmax = int(ctx.max())
    S = w.num_seqs
    k = np.zeros((S, w.num_kv_heads, lmax, w.head_dim), synth.STORAGE[w.dtype])
    v = np.zeros_like(k)
    for s, (a, b) in enumerate(w.token_streams()):
        k[s, :, :a.shape[0]] = a.transpose(1, 0, 2)
        v[s, :, :b.shape[0]] = b.transpose(1, 0, 2)
    kd = [to_device(k, dt, dev)]
    vd = [to_device(v, dt, dev)]
    del k, v
    for _ in range(args.replicas - 1):
        kd.append(kd[0].clone())
        vd.append(vd[0].clone())
    q = to_device(w.q, dt, dev)
    out = torch.empty_like(q)
    cd = torch.from_numpy(ctx).to(dev)
    ws = kernels.alloc_workspace(S, w.num_q_heads, w.head_dim, lmax, P, dev)
    stream = torch.cuda.current_stream()
    n = max(20, args.steps)
    for i in range(10):
        kernels.contiguous_attention_decode(out, q, kd[i % args.replicas], vd[i % args.replicas], cd, lmax, w.scale, P,
                                            ws, args.flags)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record(stream)
        kernels.contiguous_attention_decode(out, q, kd[i % args.replicas], vd[i % args.replicas], cd, lmax, w.scale, P,
                                            ws, args.flags)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    us = 1e3 * sum(a.elapsed_time(b) for a, b in evs) / n
    return {"attention_us": round(us, 2), "paged_over_contiguous": round(paged_us / us - 1.0, 4)}


def cpu_baseline(w, P, a_bytes, seconds):
    """The oracle (plain fp64 C, OpenMP over (sequence, head)) on the host cores, same workload."""
    import oracle

    st = oracle.replay(w, attend_checks=False)
    reps, t = 0, 0.0
    t0 = time.perf_counter()
    while t < seconds or reps == 0:
        oracle.attention_of(st, w, P)
        reps += 1
        t = time.perf_counter() - t0
    per_call = t / reps
    return {"value": round(a_bytes / per_call / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle", "sample": f"the full {w.name} batch ({w.num_seqs} sequences), {reps} calls in "
                                        f"{t:.1f} s, {per_call * 1e3:.1f} ms per call",
            "decode_tokens_per_s": round(w.num_seqs / per_call, 2)}


if __name__ == "__main__":
    main()
