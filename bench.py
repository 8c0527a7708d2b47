#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV cache on one MI355X.

One step = the decode step's device work on inputs resident in HBM:
  reshape_and_cache (write each sequence's new token into its slot)
  + paged_attention_decode (one query token per sequence over its paged context)
on the 13B-shaped workload by default (40 heads x 128, fp16, block 16, 30 sequences,
context U[128, 2048]). Slot assignment for the step is done once by the host allocator
before timing.

Prints ONE JSON line. GB/s counts algorithmic bytes: each context token's K and V rows once
(for shared blocks, each physical block once: the unique bytes), q in, out, table entries and
lengths; plus the new tokens' K/V read and written by reshape_and_cache.

Helper modes (no GPU needed) turn rocprofv3 CSV output into the short text summaries kept
under profiles/:
  bench.py --summarize-trace KERNEL_STATS_CSV OUT_TXT "COMMAND"
  bench.py --summarize-counters WORKLOAD_NAME FETCH_CSV WRITE_CSV OUT_TXT "FETCH_COMMAND" "WRITE_COMMAND"
"""
import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV GB/s (% HBM peak) and decode tokens/s, 13B shape"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
PARTITION_BALANCED = -1  # the library's balanced split mode
FLAG_CACHED_KV = 2  # the library's cached K/V load flag
PROFILES = os.path.join(ROOT, "profiles")
CSRC = "paged_kv_cache_416_amd/csrc/"
# counter summaries under profiles/: name -> (workload, sources of its attention kernel, kernel name
# part, partition size, flags and cached-load hint the summary was taken at)
_GQA_SOURCES = [CSRC + "attention_gqa.hip", CSRC + "mfma.h", CSRC + "attention.h", CSRC + "common.h"]
COUNTERS = {
    "attn_decode_f16_13b_counters.txt": ("13b-decode", [CSRC + "attention.hip", CSRC + "attention.h", CSRC + "common.h"],
                                         "attn_decode_kernel", 0, 0, "none"),
    "attn_gqa_bf16_8b_balanced_counters.txt": ("8b-gqa-prefix", _GQA_SOURCES, "attn_gqa_balanced_kernel",
                                               PARTITION_BALANCED, 0, "shared"),
    "attn_gqa_bf16_8b_p512_counters.txt": ("8b-gqa-prefix", _GQA_SOURCES, "attn_gqa_parts_kernel", 512, 0, "shared"),
}


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def attention_bytes(ctx, hq, hkv, d, elt, bs, unique_blocks=None):
    """Algorithmic bytes of one decode-attention call: (logical, unique).

    logical: every sequence's K and V rows; unique: each physical block's rows once, at the
    number of rows the longest sequence mapping it uses (equal to logical without sharing)."""
    kv_row = 2 * hkv * d * elt
    logical_kv = sum(int(c) for c in ctx) * kv_row
    unique_kv = logical_kv if unique_blocks is None else sum(unique_blocks.values()) * kv_row
    other = 2 * len(ctx) * hq * d * elt + sum(-(-int(c) // bs) for c in ctx) * 4 + 4 * len(ctx)
    return logical_kv + other, unique_kv + other


def unique_rows(tables, ctx, bs):
    """Physical block -> rows used, over all sequences (shared blocks counted once)."""
    rows = {}
    for t, c in zip(tables, ctx):
        c = int(c)
        for j in range(-(-c // bs)):
            b = int(t[j])
            rows[b] = max(rows.get(b, 0), min(bs, c - j * bs))
    return rows


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="13b", choices=["13b", "sweep-b8", "sweep-b16", "sweep-b32", "gqa"])
    ap.add_argument("--partition", default="default",
                    help="partition size in tokens, 0 (single pass), 'balanced', or 'default' (the workload's)")
    ap.add_argument("--replicas", type=int, default=3, help="cache copies rotated across steps (defeats the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-contiguous", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true")
    ap.add_argument("--no-gqa-leg", action="store_true",
                    help="with the 13B workload, skip the 8B-shaped grouped-query legs (decode: gqa_8b; and the "
                         "default prefill leg)")
    ap.add_argument("--swap", action="store_true", help="also time preemption by swap (device <-> pinned host)")
    ap.add_argument("--no-cache-ops-leg", action="store_true",
                    help="with the 13B workload, skip the cache-write legs (copy_blocks, reshape_and_cache)")
    ap.add_argument("--prefix-cache", action="store_true", help="also time the host prefix cache")
    ap.add_argument("--prefill", type=int, default=None, metavar="PROMPT_LEN",
                    help="also time paged prefill of 8 prompts of this length (8B shape); 0 skips it. Default: "
                         "2048 with the 13B workload and its grouped-query legs, else skipped")
    ap.add_argument("--memory-sim", action="store_true",
                    help="host only: run the continuous-batching memory simulator and print its JSON line")
    ap.add_argument("--cpu-one-thread", nargs=2, metavar=("WORKLOAD", "PARTITION"), help=argparse.SUPPRESS)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--flags", type=int, default=-1, help="attention flags; -1 = the workload's default")
    ap.add_argument("--step", choices=["fused", "separate"], default="fused",
                    help="a decode step as one call (pkv_paged_attention_decode_step) or as the two calls")
    ap.add_argument("--cached-lens", choices=["default", "none", "shared"], default="default",
                    help="cached-load hint: none, or each sequence's shared prefix from the reference counts")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after timing, run a plain elementwise kernel over this many MiB (counter calibration)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("STATS_CSV", "OUT", "CMD"))
    ap.add_argument("--summarize-counters", nargs=6,
                    metavar=("WORKLOAD_NAME", "FETCH_CSV", "WRITE_CSV", "OUT", "CMD1", "CMD2"))
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ARG",
                    help="OUT KERNEL_PART TITLE CSV CMD [CSV CMD ...]: per-dispatch means of every counter of "
                         "rocprofv3 --pmc passes for the kernels whose name contains KERNEL_PART")
    return ap.parse_args()


# layers of the model each workload is shaped after (the attention-only tokens/s figure)
LAYERS = {"13b-decode": 40, "8b-gqa-prefix": 32}


def make_workload(name):
    """(workload, default partition size, default flags)."""
    import synth
    if name == "13b":
        return synth.llama13b(), 0, 0
    if name.startswith("sweep-b"):
        return synth.block_sweep(block_size=int(name[7:])), 0, 0
    if name == "gqa":
        # every sequence maps the same 1024-token prefix blocks; the reference counts give each
        # sequence's shared prefix, which is loaded through the caches (the default cached-load
        # hint of this workload), the private blocks non-temporally
        return synth.gqa_shared_prefix(), 512, 0
    raise ValueError(name)


def kernel_label(w, P, flags):
    """Names of the kernels one attention call launches (the library's dispatch rule)."""
    g = w.num_q_heads // w.num_kv_heads
    mfma = (g > 1 and w.dtype in ("f16", "bf16") and w.head_dim == 128 and w.block_size in (16, 32)
            and g <= 16 and not flags & 1)
    if P == PARTITION_BALANCED:
        return ("attn_gqa_balanced_kernel" if mfma else "attn_decode_balanced_kernel") + "+attn_reduce_balanced_kernel"
    if mfma and P > 0 and len(w.batch) <= 4096:  # the persistent fixed-partition schedule
        return "attn_gqa_parts_kernel+attn_gqa_reduce_parts_kernel"
    if mfma:
        return "attn_gqa_mfma_kernel" + ("+attn_gqa_reduce_kernel" if P > 0 else "")
    return "attn_decode_kernel" + ("+attn_reduce_kernel" if P > 0 else "")


def launch_percentiles(fn, n, stream):
    """p10 / p50 / p90 of single-launch device times of fn(i): an event on the launch stream
    before every launch and after the last (each interval holds one launch and its gap)."""
    import numpy as np
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    for i in range(n):
        ev[i].record(stream)
        fn(i)
    ev[n].record(stream)
    torch.cuda.synchronize()
    d = np.array([1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    return {f"p{q}": round(float(np.percentile(d, q)), 2) for q in (10, 50, 90)}


def timed_launches(fn, n, stream):
    """Average device time of one launch of fn(i): HIP events on the launch stream around n
    back-to-back launches (the gaps between them included)."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / n


def read_counters(workload, P, flags, hint):
    """Measured HBM bytes per attention launch from the committed counter summary taken on this
    workload at this partition size, flags and cached-load hint, on the kernel source as it is
    now; else None."""
    for fname, entry in COUNTERS.items():
        if entry[0] != workload or (P, flags, hint) != (entry[3], entry[4], entry[5]):
            continue
        path = os.path.join(PROFILES, fname)
        if not os.path.exists(path):
            return None
        kv = {}
        with open(path) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != source_hash(entry[1]):
            return None
        return float(kv["traffic_bytes_per_dispatch"])
    return None


class Setup:
    """One workload's device state for timing: the cache built by every op but the decode step's own
    append, `replicas` copies of the caches, the step's new rows and slots, tables and queries."""

    def __init__(self, w, args, dev, hint):
        import numpy as np
        import torch

        from paged_kv_cache_416_amd.cache import PagedKVCache, run_ops, to_device

        self.w, self.dev = w, dev
        self.dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        dt, B = self.dt, w.block_size
        cache = PagedKVCache(w.num_blocks, B, w.num_kv_heads, w.head_dim, dt, device=dev, free_order=w.free_order)
        run_ops(cache, w.ops[:-1], dt)
        step = w.ops[-1][1]  # [(sid, k[1,Hkv,D], v[1,Hkv,D]), ...]
        slots, pairs = cache.pool.append([(sid, k.shape[0]) for sid, k, _ in step])
        assert len(pairs) == 0
        # a step's new rows in batch order (one token per sequence), for the one-launch step
        assert [sid for sid, _, _ in step] == list(w.batch)
        self.cache = cache
        self.n_new = len(step)
        self.new_k = to_device(np.concatenate([k for _, k, _ in step]), dt, dev)
        self.new_v = to_device(np.concatenate([v for _, _, v in step]), dt, dev)
        self.slot_dev = torch.from_numpy(slots).to(dev)
        self.tb_host, self.ctx_host = cache.pool.tables(w.batch)
        self.tb = torch.from_numpy(self.tb_host).to(dev)
        self.ctx_dev = torch.from_numpy(self.ctx_host).to(dev)
        self.max_ctx = int(self.ctx_host.max())
        self.hint = hint
        self.cached_lens = cache.shared_prefix_lens(w.batch) if hint == "shared" else None
        self.ctx = w.final_lengths()
        self.q = to_device(w.q, dt, dev)
        self.out = torch.empty_like(self.q)
        self.replicas = args.replicas
        self.ks = [cache.k] + [cache.k.clone() for _ in range(args.replicas - 1)]
        self.vs = [cache.v] + [cache.v.clone() for _ in range(args.replicas - 1)]
        torch.cuda.synchronize()
        elt = w.elt_bytes
        self.logical_b, self.unique_b = attention_bytes(self.ctx, w.num_q_heads, w.num_kv_heads, w.head_dim, elt, B,
                                                        unique_rows(self.tb_host, self.ctx_host, B))
        # K1: read + write K and V of each new token, and its slot
        self.w_bytes = 2 * 2 * self.n_new * w.num_kv_heads * w.head_dim * elt + 8 * self.n_new


def measure(st, P, flags, args, step_mode, percentiles=True):
    """Time one workload in one split mode: whole decode steps (host clock, `steps` steps after
    `warmup`), the other step form, and the attention launches alone (HIP events on the launch
    stream) for the roofline."""
    import torch

    from paged_kv_cache_416_amd import kernels

    w = st.w
    S, hq, d = w.num_seqs, w.num_q_heads, w.head_dim
    ws = kernels.alloc_workspace(S, hq, d, st.max_ctx, P, st.dev)
    stream = torch.cuda.current_stream()
    R = st.replicas

    def attend(i):
        r = i % R
        kernels.paged_attention_decode(st.out, st.q, st.ks[r], st.vs[r], st.tb, st.ctx_dev, st.max_ctx, w.scale, P, ws,
                                       flags, st.cached_lens)

    def separate_step(i):
        r = i % R
        kernels.reshape_and_cache(st.new_k, st.new_v, st.ks[r], st.vs[r], st.slot_dev)
        attend(i)

    def fused_step(i):
        r = i % R
        kernels.paged_attention_decode_step(st.out, st.q, st.new_k, st.new_v, st.slot_dev, st.ks[r], st.vs[r], st.tb,
                                            st.ctx_dev, st.max_ctx, w.scale, P, ws, flags, st.cached_lens)

    def time_steps(fn, steps):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        # timed region: exactly `steps` whole steps, synchronised on both sides, host clock
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    one_step, other_step = (fused_step, separate_step) if step_mode == "fused" else (separate_step, fused_step)
    # both forms run before either is timed: the first timed loop of a process otherwise runs
    # about 1 % slow (measured with either form first), which would favour the second
    for i in range(args.warmup):
        other_step(i)
        one_step(i)
    ms_per_step = time_steps(one_step, args.steps)
    ms_other = time_steps(other_step, args.steps)
    # the attention launches alone, for the roofline
    attn_us = timed_launches(attend, args.steps, stream)
    value = (st.unique_b + st.w_bytes) / (ms_per_step * 1e-3) / 1e9
    achieved = st.unique_b / (attn_us * 1e-6) / 1e9
    traffic = read_counters(w.name, P, flags, st.hint)
    res = {
        "ms_per_step": ms_per_step,
        "ms_other": ms_other,
        "value": value,
        "attention_us": attn_us,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": round(traffic) if traffic is not None else None,
                     "kernel": kernel_label(w, P, flags)},
    }
    if percentiles:
        res["attention_us_single_launch"] = launch_percentiles(attend, max(100, args.steps), stream)
    return res


def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(*args.summarize_trace)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)
    if args.summarize_pmc:
        a = args.summarize_pmc
        return summarize_pmc(a[0], a[1], a[2], list(zip(a[3::2], a[4::2])))
    if args.cpu_one_thread:
        return cpu_one_thread(args.cpu_one_thread[0], int(args.cpu_one_thread[1]))
    if args.memory_sim:
        print(json.dumps(memory_sim_leg()))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported. The path shards by sequence or by "
              f"KV head with no exchange between GPUs, so one GPU's figure at its share of the batch is the "
              f"per-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w, default_P, default_flags = make_workload(args.workload)
    flags = default_flags if args.flags < 0 else args.flags
    hint = args.cached_lens if args.cached_lens != "default" else ("shared" if args.workload == "gqa" else "none")
    step_mode = args.step
    P = {"default": default_P, "balanced": PARTITION_BALANCED}.get(args.partition)
    if P is None:
        P = int(args.partition)
    st = Setup(w, args, dev, hint)
    S, hq, hkv, d, B = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    m = measure(st, P, flags, args, step_mode)
    ms_per_step, attn_us, value = m["ms_per_step"], m["attention_us"], m["value"]
    ctx = st.ctx

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
        "data": "synthetic (seeded N(0,1)*0.5 keys/values, seeded context lengths and physical block order)",
        "config": {"workload": w.name, "num_seqs": S, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
                   "block_size": B, "sum_context": int(ctx.sum()), "max_context": int(ctx.max()),
                   "partition_size": P, "flags": flags, "cached_lens": hint, "step": step_mode,
                   "replicas": args.replicas},
        "pct_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "decode_tokens_per_s": round(S / (ms_per_step * 1e-3), 1),
        "decode_tokens_per_s_attention_only": {
            "layers": LAYERS.get(w.name, 40),
            "value": round(S / (LAYERS.get(w.name, 40) * attn_us * 1e-6), 1)},
        "ms_per_step_" + ("separate" if step_mode == "fused" else "fused"): round(m["ms_other"], 5),
        "attention_us": round(attn_us, 2),
        "attention_us_single_launch": m["attention_us_single_launch"],
        "bytes_per_step": {"attention_logical": st.logical_b, "attention_unique": st.unique_b,
                           "cache_write": st.w_bytes},
        "roofline": m["roofline"],
    }
    unique_b = st.unique_b
    cache = st.cache
    dt = st.dt

    if args.copy_probe:
        # a plain elementwise kernel that reads and writes a known number of bytes, by which the
        # HBM byte counters are calibrated (its kernel name contains "neg")
        src = torch.empty(args.copy_probe << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
        del src, dst

    if not args.no_read_probe:
        result["stream_read"] = read_probe_leg(unique_b, args, dev)

    if not args.no_contiguous:
        result["contiguous"] = contiguous_leg(w, P, args, dev, dt, attn_us, flags)

    if args.swap:
        result["swap"] = swap_leg(cache, w, dev, dt)

    if args.prefix_cache:
        result["prefix_cache"] = prefix_cache_leg()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.workload, P, unique_b, args.cpu_seconds)

    if args.workload == "13b" and not args.no_gqa_leg:
        del st, cache
        torch.cuda.empty_cache()
        result["gqa_8b"] = gqa_leg(args, dev, with_cpu=not args.no_cpu_baseline)

    if args.workload == "13b" and not args.no_cache_ops_leg:
        result["cache_ops"] = cache_ops_leg(dev)

    prefill_len = args.prefill
    if prefill_len is None:
        prefill_len = 2048 if args.workload == "13b" and not args.no_gqa_leg else 0
    if prefill_len:
        result["prefill"] = prefill_leg(dev, prefill_len)

    print(json.dumps(result), flush=True)


def gqa_leg(args, dev, with_cpu=True):
    """The 8B-shaped grouped-query workload (32 query / 8 KV heads, bf16, 256 sequences over a shared
    1024-token prefix): whole decode steps and the attention launches at its configured split
    (partitions of 512 tokens, then the merge pass) and in the balanced mode, each with its own
    roofline on unique bytes (each physical block once); the oracle on the same batch beside it."""
    w, P_cfg, flags = make_workload("gqa")
    st = Setup(w, args, dev, "shared")
    res = {"workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
           "head_dim": w.head_dim, "block_size": w.block_size, "dtype": w.dtype, "sum_context": int(st.ctx.sum()),
           "max_context": int(st.ctx.max()), "cached_lens": "shared",
           "bytes_per_step": {"attention_logical": st.logical_b, "attention_unique": st.unique_b,
                              "cache_write": st.w_bytes}}
    for label, P in (("configured_split", P_cfg), ("balanced", PARTITION_BALANCED)):
        m = measure(st, P, flags, args, "fused", percentiles=False)
        res[label] = {"partition_size": P, "ms_per_step": round(m["ms_per_step"], 5),
                      "value": round(m["value"], 2), "unit": "GB/s",
                      "pct_hbm_peak": round(100 * m["value"] / PEAK_HBM_GBS, 2),
                      "attention_us": round(m["attention_us"], 2),
                      "decode_tokens_per_s": round(w.num_seqs / (m["ms_per_step"] * 1e-3), 1),
                      "decode_tokens_per_s_attention_only": {
                          "layers": LAYERS[w.name],
                          "value": round(w.num_seqs / (LAYERS[w.name] * m["attention_us"] * 1e-6), 1)},
                      "roofline": m["roofline"]}
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(w, "gqa", P_cfg, st.unique_b, args.cpu_seconds / 2, one_thread=False)
    return res


def swap_leg(cache, w, dev, dt, reps=5):
    """Preemption by swap at this shape: the newest third of the batch moves to a pinned host pool
    (pkv_seq_migrate + pkv_swap_blocks) and back, `reps` round trips; GB/s of block bytes moved
    each way, next to the runtime's own pinned-host copies of the same byte count."""
    import torch

    from paged_kv_cache_416_amd import Pool, kernels
    victims = list(w.batch[-max(1, len(w.batch) // 3):])
    nblk = len({b for s in victims for b in cache.pool.blocks(s)})
    host = Pool(nblk, w.block_size)
    shape = (nblk,) + tuple(cache.k.shape[1:])
    hk = torch.empty(shape, dtype=dt).pin_memory()
    hv = torch.empty(shape, dtype=dt).pin_memory()
    stream = torch.cuda.current_stream()
    block_bytes = cache.k[0].numel() * cache.k.element_size()
    t_out, t_in = [], []
    for _ in range(reps):
        for src_pool, dst_pool, src, dst, acc in ((cache.pool, host, [cache.k, cache.v], [hk, hv], t_out),
                                                  (host, cache.pool, [hk, hv], [cache.k, cache.v], t_in)):
            pairs = src_pool.migrate(dst_pool, victims)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            kernels.swap_blocks(src, dst, pairs)
            b.record(stream)
            torch.cuda.synchronize()
            acc.append(1e3 * a.elapsed_time(b))
    nbytes = 2 * nblk * block_bytes
    flat_h = torch.empty(nbytes // 2, dtype=torch.int16).pin_memory()
    flat_d = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)

    def copy_us(dst_t, src_t):
        dst_t.copy_(src_t, non_blocking=True)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            dst_t.copy_(src_t, non_blocking=True)
        b.record(stream)
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / reps

    d2h, h2d = copy_us(flat_h, flat_d), copy_us(flat_d, flat_h)
    out_us, in_us = sorted(t_out)[len(t_out) // 2], sorted(t_in)[len(t_in) // 2]
    return {"sequences": len(victims), "blocks": nblk, "bytes": nbytes,
            "out_us": round(out_us, 1), "out_GB/s": round(nbytes / out_us / 1e3, 1),
            "in_us": round(in_us, 1), "in_GB/s": round(nbytes / in_us / 1e3, 1),
            "runtime_copy_GB/s": {"device_to_host": round(nbytes / d2h / 1e3, 1),
                                  "host_to_device": round(nbytes / h2d / 1e3, 1)}}


def prefix_cache_leg(requests=256, system=1024, seed=11):
    """Host cost of the prefix cache at the 8B-shaped GQA workload's shape: `requests` prompts
    opening with one shared `system`-token prompt plus lognormal private tails, added through
    pkv_seq_add_prompt (chained SHA-256 per full block, lookup, allocation)."""
    import numpy as np

    from paged_kv_cache_416_amd import Pool
    rng = np.random.default_rng(seed)
    tails = np.clip(np.round(np.exp(rng.normal(np.log(1024), 1.0, size=requests))), 1, 8192).astype(np.int64)
    sys_toks = rng.integers(0, 128000, size=system).astype(np.int32)
    prompts = [np.concatenate([sys_toks, rng.integers(0, 128000, size=int(t)).astype(np.int32)]) for t in tails]
    B = 16
    pool = Pool(int(sum(-(-len(p) // B) for p in prompts)) + 8, B)
    cached = 0
    t0 = time.perf_counter()
    for i, p in enumerate(prompts):
        _, n = pool.add_prompt(i, p)
        cached += n
    t = time.perf_counter() - t0
    total = int(sum(len(p) for p in prompts))
    return {"requests": requests, "prompt_tokens": total, "cached_tokens": cached,
            "cached_fraction": round(cached / total, 4), "host_us_per_request": round(1e6 * t / requests, 1),
            "hashed_MB_per_s": round(total * 4 / t / 1e6, 1)}


# Memory of one token's keys and values in a 13B-class model, fp16: 2 (K, V) x 5120 x 40 layers x 2 B
# (slide 5 of the "vLLM and PagedAttention" deck).
KV_TOKEN_BYTES_13B = 2 * 5120 * 40 * 2


def memory_sim_leg(seed=7, block_size=16, reserve=2048, oracle_requests=400):
    """Continuous-batching memory simulator (host only) on two memory budgets for a 13B-class
    model: the pages' device (30 % of 40 GB for keys and values, slide 4) and one MI355X (288 GB
    less 26 GB of fp16 weights and 10 GB kept for activations). The same seeded requests
    (log-normal prompt and output lengths, medians 160 and 200 tokens, within a 2048-token
    context) all wait at step 0; the contiguous scheme reserves the whole 2048-token context per
    request (the lesson note's example), the paged scheme takes 16-slot blocks with 1 % of the
    pool kept free at admission. Reports the useful share of held memory, the batch size, the
    native simulator's cost per step, and the oracle simulator timed beside it on a sample."""
    import numpy as np

    import synth
    from oracle import simulator as ref
    from paged_kv_cache_416_amd import sim
    budgets = []
    for name, kv_bytes, n, max_batch in (("40GB-device-13B", 0.30 * 40e9, 2000, 256),
                                         ("mi355x-288GB-13B", 288e9 - 26e9 - 10e9, 20000, 4096)):
        blocks = int(kv_bytes // (KV_TOKEN_BYTES_13B * block_size))
        slots = blocks * block_size
        watermark = -(-blocks // 100)
        a, p, o = synth.serving_requests(seed, n, 160, 200, 1.0, reserve, None)
        entry = {"workload": name, "kv_bytes": int(kv_bytes), "slots": slots, "block_size": block_size,
                 "watermark_blocks": watermark, "max_batch": max_batch, "requests": n,
                 "mean_prompt": round(float(p.mean()), 1), "mean_output": round(float(o.mean()), 1),
                 "contiguous_reserve": reserve}
        for kind in ("paged", "contiguous"):
            t0 = time.perf_counter()
            if kind == "paged":
                trace, _ = sim.simulate_paged(blocks, block_size, watermark, max_batch, a, p, o, max_steps=1 << 21)
            else:
                trace, _ = sim.simulate_contiguous(slots, max_batch, a, p, o, np.full(n, reserve), max_steps=1 << 21)
            dt = time.perf_counter() - t0
            summary = sim.summarize(trace, slots)
            summary = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in summary.items()}
            summary["native_us_per_step"] = round(1e6 * dt / len(trace), 2)
            entry[kind] = summary
        budgets.append(entry)
    # the oracle beside the native simulator, on the first requests of the first budget
    c = budgets[0]
    a, p, o = synth.serving_requests(seed, c["requests"], 160, 200, 1.0, reserve, None)
    a, p, o = a[:oracle_requests], p[:oracle_requests], o[:oracle_requests]
    args = (c["slots"] // block_size, block_size, c["watermark_blocks"], c["max_batch"], a, p, o)
    t0 = time.perf_counter()
    nat, _ = sim.simulate_paged(*args)
    t_nat = time.perf_counter() - t0
    t0 = time.perf_counter()
    rows, _ = ref.simulate_paged(*args)
    t_ref = time.perf_counter() - t0
    return {"metric": "continuous-batching memory simulator: useful share of held KV memory, paged vs contiguous "
                      "reservation",
            "data": "synthetic (seeded log-normal prompt/output lengths, all requests waiting at step 0)",
            "budgets": budgets,
            "oracle": {"sample": f"paged scheme, first {oracle_requests} requests of {c['workload']}",
                       "steps": len(rows), "native_ms": round(1e3 * t_nat, 2), "oracle_ms": round(1e3 * t_ref, 1),
                       "identical": bool(np.array_equal(nat, np.array(rows, dtype=np.int64)))}}


def prefill_leg(dev, prompt_len, seqs=8, hq=32, hkv=8, d=128, B=16, reps=30, warmup=100):
    """Paged prefill at the 8B shape: `seqs` fresh prompts of `prompt_len` tokens, every token a
    causal query over the paged cache (random placement). Algorithmic flops: 4 d per (query,
    visible key, query head): q.k and p.v."""
    import numpy as np
    import torch

    from paged_kv_cache_416_amd import kernels
    rng = np.random.default_rng(21)
    nb_seq = -(-prompt_len // B)
    N = seqs * nb_seq + 16
    perm = rng.permutation(N).astype(np.int32)
    tables = torch.from_numpy(perm[:seqs * nb_seq].reshape(seqs, nb_seq).copy()).to(dev)
    k = (torch.randn(N, hkv, B, d, device=dev) * 0.5).to(torch.bfloat16)
    v = (torch.randn(N, hkv, B, d, device=dev) * 0.5).to(torch.bfloat16)
    ctx = torch.full((seqs,), prompt_len, dtype=torch.int32, device=dev)
    qs = torch.arange(0, (seqs + 1) * prompt_len, prompt_len, dtype=torch.int32, device=dev)
    q = (torch.randn(seqs * prompt_len, hq, d, device=dev) * 0.5).to(torch.bfloat16)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def run(i):
        kernels.paged_attention_prefill(out, q, k, v, tables, ctx, qs, prompt_len, prompt_len, d ** -0.5)

    # a long warm-up, at least `warmup` launches and half a second of them: after the other legs'
    # host-side work (the prefix cache, the oracle) the device comes back at lower clocks, and the
    # first tens of milliseconds of launches run several per cent slow
    t0, i = time.perf_counter(), 0
    while i < warmup or time.perf_counter() - t0 < 0.5:
        run(i)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    us = timed_launches(run, reps, stream)
    flops = 4 * d * hq * seqs * prompt_len * (prompt_len + 1) / 2
    tf = flops / (us * 1e-6) / 1e12
    return {"sequences": seqs, "prompt_len": prompt_len, "q_heads": hq, "kv_heads": hkv, "dtype": "bf16",
            "us": round(us, 1), "TFLOP/s": round(tf, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": 2500.0, "unit": "TFLOP/s",
                         "frac": round(tf / 2500.0, 4), "traffic": None},
            "tokens_per_s": round(seqs * prompt_len / (us * 1e-6), 0)}


def cache_ops_leg(dev, heads=40, d=128, B=16, pairs=2048, tokens=16384, reps=50):
    """The cache writes at the 13B shape (fp16, 40 kv heads x 128), at sizes where HBM bounds them:
    copy_blocks of `pairs` copy-on-write pairs (distinct random sources and destinations in an
    8192-block pool) and reshape_and_cache of a `tokens`-token chunk into its sequence's blocks
    (random block order, consecutive slots within a block, as a prefill writes them). Algorithmic
    bytes: every block or row read once and written once, K and V."""
    import numpy as np
    import torch

    from paged_kv_cache_416_amd import kernels
    rng = np.random.default_rng(77)
    N = 8192
    k = torch.zeros(N, heads, B, d, dtype=torch.float16, device=dev)
    v = torch.zeros_like(k)
    block_bytes = heads * B * d * 2
    stream = torch.cuda.current_stream()
    perm = rng.permutation(N).astype(np.int32)
    pair = np.stack([perm[:pairs], perm[pairs:2 * pairs]], axis=1)
    for _ in range(5):
        kernels.copy_blocks([k], [v], pair)
    cb_us = timed_launches(lambda i: kernels.copy_blocks([k], [v], pair), reps, stream)
    cb_bytes = 2 * 2 * pairs * block_bytes
    nblk = tokens // B
    table = rng.permutation(N)[:nblk].astype(np.int64)
    slots = torch.from_numpy(np.repeat(table * B, B) + np.tile(np.arange(B), nblk)).to(dev)
    key = (torch.randn(tokens, heads, d, device=dev) * 0.5).to(torch.float16)
    val = (torch.randn(tokens, heads, d, device=dev) * 0.5).to(torch.float16)
    for _ in range(5):
        kernels.reshape_and_cache(key, val, k, v, slots)
    rc_us = timed_launches(lambda i: kernels.reshape_and_cache(key, val, k, v, slots), reps, stream)
    rc_bytes = 2 * 2 * tokens * heads * d * 2 + tokens * 8

    def entry(us, nbytes, what):
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"what": what, "us": round(us, 2), "bytes": nbytes, "GB/s": round(gbs, 1),
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}}
    return {"copy_blocks": entry(cb_us, cb_bytes, f"{pairs} block pairs, K and V, 13B shape"),
            "reshape_and_cache": entry(rc_us, rc_bytes, f"{tokens} tokens into their blocks, 13B shape")}


def read_probe_leg(nbytes, args, dev):
    """The device's streaming-read rate on the attention's byte count: the library's read probe
    over `replicas` rotated buffers of that size (the same cache-defeating scheme as the caches)."""
    import torch

    from paged_kv_cache_416_amd import kernels
    n = -(-nbytes // 16) * 16
    bufs = [torch.ones(n // 4, dtype=torch.float32, device=dev) for _ in range(args.replicas)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def probe(i):
        kernels.read_probe(bufs[i % len(bufs)], sink)

    for i in range(5):
        probe(i)
    us = timed_launches(probe, max(50, args.steps), stream)
    del bufs
    return {"bytes": n, "us": round(us, 2), "GB/s": round(n / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * n / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2)}


def contiguous_leg(w, P, args, dev, dt, paged_us, flags):
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

    def attend(i):
        r = i % args.replicas
        kernels.contiguous_attention_decode(out, q, kd[r], vd[r], cd, lmax, w.scale, P, ws, flags & ~FLAG_CACHED_KV)

    for i in range(10):
        attend(i)
    us = timed_launches(attend, max(20, args.steps), stream)
    return {"attention_us": round(us, 2), "paged_over_contiguous": round(paged_us / us - 1.0, 4)}


def cpu_baseline(w, workload, P, a_bytes, seconds, one_thread=True):
    """The oracle (plain fp64 C, OpenMP over (sequence, head)) on the host cores, same workload;
    and (one_thread) one call of it on one thread, in a child process started with OMP_NUM_THREADS=1."""
    import subprocess

    import oracle

    st = oracle.replay(w, attend_checks=False)
    reps, t = 0, 0.0
    t0 = time.perf_counter()
    while t < seconds or reps == 0:
        oracle.attention_of(st, w, P)
        reps += 1
        t = time.perf_counter() - t0
    per_call = t / reps
    res = {"value": round(a_bytes / per_call / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
           "kind": "oracle", "sample": f"the full {w.name} batch ({w.num_seqs} sequences), {reps} calls in "
                                       f"{t:.1f} s, {per_call * 1e3:.1f} ms per call",
           "decode_tokens_per_s": round(w.num_seqs / per_call, 2), "cpu_model": cpu_model()}
    if not one_thread:
        return res
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-one-thread", workload, str(P)], env=env,
                       capture_output=True, text=True, timeout=300)
    if r.returncode == 0 and r.stdout.strip():
        one = json.loads(r.stdout.strip().splitlines()[-1])
        res["one_thread"] = {"threads": one["threads"], "value": round(a_bytes / one["s_per_call"] / 1e9, 3),
                             "ms_per_call": round(one["s_per_call"] * 1e3, 1)}
    else:
        res["one_thread"] = {"error": (r.stderr or "no output").strip().splitlines()[-1][:200]}
    return res


def cpu_one_thread(workload, P):
    """Child-process side of cpu_baseline: one oracle call on the workload (no GPU use)."""
    import oracle
    w, _, _ = make_workload(workload)
    st = oracle.replay(w, attend_checks=False)
    t0 = time.perf_counter()
    oracle.attention_of(st, w, P)
    print(json.dumps({"threads": oracle.threads(), "s_per_call": time.perf_counter() - t0}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------------- profile summaries (no GPU)

def _short(name):
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0][:110]


def summarize_trace(stats_csv, out, cmd):
    """rocprofv3 --kernel-trace --stats kernel table -> a short text summary."""
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel-trace summary (durations in microseconds)",
             f"# command: {cmd}",
             f"{'kernel':<112} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for r in rows:
        lines.append(f"{_short(r['Name']):<112} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                     f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>6.2f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(workload, fetch_csv, write_csv, out, cmd_fetch, cmd_write):
    """Two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) -> HBM bytes per attention
    launch, each counter scaled by what it reads for a plain elementwise kernel over a known size."""
    def per_kernel(path):
        acc = {}
        for r in csv.DictReader(open(path)):
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    probe = [k for k in fetch if "neg_kernel" in k]
    _, sources, kname, _, _, _ = COUNTERS[os.path.basename(out)]
    attn = [k for k in fetch if kname in k]
    if len(probe) != 1 or len(attn) != 1:
        raise SystemExit(f"expected one probe and one attention kernel, got {probe} / {attn}")
    probe_bytes = 1 << 30  # --copy-probe 1024: 1 GiB read, 1 GiB written
    pf, pw = max(fetch[probe[0]]), max(write[probe[0]])
    fs, wsc = probe_bytes / (pf * 1024), probe_bytes / (pw * 1024)
    af = sum(fetch[attn[0]]) / len(fetch[attn[0]])
    aw = sum(write[attn[0]]) / len(write[attn[0]])
    traffic = af * 1024 * fs + aw * 1024 * wsc
    lines = ["# HBM bytes of the attention kernel, from two rocprofv3 --pmc passes (counters in KiB per dispatch)",
             f"# command (FETCH_SIZE): {cmd_fetch}",
             f"# command (WRITE_SIZE): {cmd_write}",
             "# scale = bytes the calibration kernel (torch.neg over 1 GiB: 1 GiB read, 1 GiB written) moved,",
             "#         divided by what the counter reported for it",
             f"kernel: {_short(attn[0])}",
             f"kernel_source_sha256: {source_hash(sources)}",
             f"dispatches: {len(fetch[attn[0]])}",
             f"fetch_kib_per_dispatch: {af:.1f}",
             f"write_kib_per_dispatch: {aw:.1f}",
             f"probe_fetch_kib: {pf:.1f}",
             f"probe_write_kib: {pw:.1f}",
             f"fetch_scale: {fs:.4f}",
             f"write_scale: {wsc:.4f}",
             f"traffic_bytes_per_dispatch: {traffic:.0f}"]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(out, kernel_part, title, passes):
    """rocprofv3 --pmc passes (one counter set each) -> the mean value per dispatch of every counter,
    for each kernel whose name contains kernel_part, with the command of each pass."""
    per = {}  # kernel -> counter -> [values]
    for path, _ in passes:
        for r in csv.DictReader(open(path)):
            if kernel_part not in r["Kernel_Name"]:
                continue
            per.setdefault(_short(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    lines = [f"# {title}", "# rocprofv3 --pmc, one pass per counter set; values are means per dispatch"]
    for path, cmd in passes:
        lines.append(f"# command: {cmd}")
    for k, cs in per.items():
        lines.append(f"kernel: {k}")
        for c, v in cs.items():
            lines.append(f"  {c}: {sum(v) / len(v):.6g}  (dispatches {len(v)})")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
