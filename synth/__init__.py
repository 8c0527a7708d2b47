"""Seeded synthetic workloads for paged decode attention.

This module only *draws* inputs: context lengths, the order in which physical
blocks leave the free pool, queries, and each logical token's key/value rows,
rounded once (round-to-nearest-even) to the storage dtype. It also writes down
the sequence of cache operations (add / append / fork / free) that builds each
workload's cache state, as plain data.

It holds none of the method's arithmetic: no slot or block-table computation,
no scatter, no attention. The GPU library and the CPU oracle both replay the
same operations with their own code, so neither depends on the other.

Streams are keyed by ``numpy.random.default_rng([seed, tag, *index])`` (PCG64
seeded through SeedSequence), so one sequence's tokens can be regenerated
without drawing any other sequence's.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

# stream tags
_LENGTHS, _FREE, _Q, _KV, _PREFIX, _PROMPT = 1, 2, 3, 4, 5, 6
_SYSTEM, _SYSKV, _TOKENS = 7, 8, 9
_REQUESTS = 10
_SCORES = 11

DTYPES = ("f32", "f16", "bf16")
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def _rng(seed, tag, *idx):
    return np.random.default_rng([int(seed), int(tag), *[int(i) for i in idx]])


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values once to the storage dtype (RNE). bf16 is kept as raw uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        nan = np.isnan(x)
        r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
        if nan.any():
            r[nan] = np.uint16(0x7FC0)
        return r
    raise ValueError(f"unknown dtype {dtype}")


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen storage values (as produced by to_storage or read back from a device) to float64."""
    if dtype == "bf16":
        a = np.ascontiguousarray(a).view(np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def normal(rng, shape, scale, dtype):
    n = int(np.prod(shape))
    x = rng.standard_normal(n, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return to_storage(x.reshape(shape), dtype)


@dataclass
class Workload:
    """One synthetic configuration.

    ``ops`` is replayed in order. Each entry is one of
      ("add", sid) | ("fork", parent, child) | ("free", sid)
      | ("append", [(sid, k, v), ...])   k, v: [n, num_kv_heads, head_dim] storage arrays
      | ("check",)                       evaluate attention for ``batch`` at this point
    The last op of a decode workload is the decode step's own append (one token per sequence).
    """

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray
    scale: float  # an exactly representable float32 value
    partition_size: int
    ops: list
    batch: list
    q: np.ndarray  # [len(batch), Hq, D] storage
    lmax: int = 0  # row capacity of the contiguous companion layout
    value_scale: float = 1.0
    notes: dict = field(default_factory=dict)

    @property
    def elt_bytes(self):
        return ELT_BYTES[self.dtype]

    @property
    def num_seqs(self):
        return len(self.batch)

    def final_lengths(self):
        """Context length of every batch sequence after all ops (bookkeeping of token counts only)."""
        n = {}
        for op in self.ops:
            if op[0] == "add":
                n[op[1]] = 0
            elif op[0] == "fork":
                n[op[2]] = n[op[1]]
            elif op[0] == "free":
                del n[op[1]]
            elif op[0] == "append":
                for sid, k, _ in op[1]:
                    n[sid] += k.shape[0]
        return np.array([n[s] for s in self.batch], dtype=np.int32)

    def token_streams(self):
        """Per batch sequence, its logical key and value rows in token order ([ctx, Hkv, D] each)."""
        rows = {}
        for op in self.ops:
            if op[0] == "add":
                rows[op[1]] = ([], [])
            elif op[0] == "fork":
                rows[op[2]] = (list(rows[op[1]][0]), list(rows[op[1]][1]))
            elif op[0] == "free":
                del rows[op[1]]
            elif op[0] == "append":
                for sid, k, v in op[1]:
                    rows[sid][0].append(k)
                    rows[sid][1].append(v)
        shp = (0, self.num_kv_heads, self.head_dim)
        out = []
        for s in self.batch:
            ks, vs = rows[s]
            out.append((np.concatenate(ks) if ks else np.zeros(shp, STORAGE[self.dtype]),
                        np.concatenate(vs) if vs else np.zeros(shp, STORAGE[self.dtype])))
        return out


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


def _draw_kv(seed, tag, keys, counts, hkv, d, vscale, dtype):
    """Draw K then V rows for each key (a stream index tuple) in parallel threads."""
    def one(i):
        r = _rng(seed, tag, *keys[i])
        k = normal(r, (counts[i], hkv, d), vscale, dtype)
        v = normal(r, (counts[i], hkv, d), vscale, dtype)
        return k, v
    with ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(one, range(len(keys))))


def _pool_size(blocks_needed, factor=1.1):
    return int(math.ceil(factor * blocks_needed))


def decode_workload(name, seed, lengths, hq, hkv, d, bs, dtype, vscale, qscale,
                     partition_size=0, lmax=0, scale=None, notes=None):
    """Independent sequences: prefill ctx-1 tokens each, then a one-token decode append."""
    lengths = np.asarray(lengths, dtype=np.int64)
    S = len(lengths)
    need = int(sum(-(-int(c) // bs) for c in lengths))
    nb = max(1, _pool_size(need))
    free_order = _rng(seed, _FREE).permutation(nb).astype(np.int32)
    q = normal(_rng(seed, _Q), (S, hq, d), qscale, dtype)
    kv = _draw_kv(seed, _KV, [(s,) for s in range(S)], [int(c) for c in lengths], hkv, d, vscale, dtype)
    ops = [("add", s) for s in range(S)]
    pre = [(s, kv[s][0][:-1], kv[s][1][:-1]) for s in range(S) if lengths[s] > 1]
    if pre:
        ops.append(("append", pre))
    last = [(s, kv[s][0][-1:], kv[s][1][-1:]) for s in range(S) if lengths[s] > 0]
    if last:
        ops.append(("append", last))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Workload(name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    block_size=bs, num_blocks=nb, free_order=free_order,
                    scale=float(np.float32(scale)), partition_size=partition_size, ops=ops,
                    batch=list(range(S)), q=q, lmax=lmax or int(lengths.max(initial=1)),
                    value_scale=vscale, notes=dict(notes or {}))


# ---------------------------------------------------------------------------
# The five configurations. Each builder takes size overrides so tests can run
# the same recipe at a reduced size.
# ---------------------------------------------------------------------------

def tiny(seed=1):
    """4 sequences, lengths {5,16,17,42}, 4 heads x 64, block 16, fp32, pool of 16 blocks."""
    lengths = [5, 16, 17, 42]
    S, H, D, B = 4, 4, 64, 16
    nb = 16
    free_order = _rng(seed, _FREE).permutation(nb).astype(np.int32)
    q = normal(_rng(seed, _Q), (S, H, D), 1.0, "f32")
    kv = _draw_kv(seed, _KV, [(s,) for s in range(S)], lengths, H, D, 1.0, "f32")
    ops = [("add", s) for s in range(S)]
    ops.append(("append", [(s, kv[s][0][:-1], kv[s][1][:-1]) for s in range(S)]))
    ops.append(("append", [(s, kv[s][0][-1:], kv[s][1][-1:]) for s in range(S)]))
    return Workload(name="tiny-fp32", dtype="f32", num_q_heads=H, num_kv_heads=H, head_dim=D,
                    block_size=B, num_blocks=nb, free_order=free_order, scale=0.125,
                    partition_size=0, ops=ops, batch=list(range(S)), q=q, lmax=64,
                    value_scale=1.0)


def llama13b(seed=2, num_seqs=30, ctx_range=(128, 2048), dtype="f16", block_size=16,
             partition_size=0):
    """13B-shaped decode: 40 heads x 128 (hidden 5120), block 16, context U[128, 2048], values N(0,1)*0.5."""
    lengths = _rng(seed, _LENGTHS).integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs)
    return decode_workload("13b-decode", seed, lengths, 40, 40, 128, block_size, dtype, 0.5, 0.5,
                            partition_size=partition_size, lmax=ctx_range[1])


def block_sweep(block_size=16, seed=4, num_seqs=64, ctx_range=(512, 4096), dtype="f16"):
    """Block-size sweep shape: 64 sequences, 40 x 128 fp16, context U[512, 4096]."""
    lengths = _rng(seed, _LENGTHS).integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs)
    return decode_workload(f"sweep-b{block_size}", seed, lengths, 40, 40, 128, block_size, dtype,
                            0.5, 0.5, lmax=ctx_range[1])


def gqa_shared_prefix(seed=5, num_seqs=256, prefix=1024, median=1024, sigma=1.0, cap=8192,
                      hq=32, hkv=8, d=128, block_size=16, dtype="bf16", partition_size=512):
    """Llama-3-8B-shaped GQA decode over a shared system-prompt prefix.

    Private length L_i = clip(round(exp(N(ln median, sigma))), 1, cap); context = prefix + L_i.
    The prefix is appended once to a template sequence, every batch sequence forks it,
    appends its private tokens (the last one as the decode step), and the template is freed.
    """
    r = _rng(seed, _LENGTHS)
    priv = np.clip(np.rint(np.exp(r.normal(math.log(median), sigma, size=num_seqs))), 1, cap).astype(np.int64)
    need = -(-prefix // block_size) + int(sum(-(-int(x) // block_size) for x in priv))
    if prefix % block_size:
        need += num_seqs  # each sequence copies the shared partial block once
    nb = _pool_size(need)
    free_order = _rng(seed, _FREE).permutation(nb).astype(np.int32)
    q = normal(_rng(seed, _Q), (num_seqs, hq, d), 0.5, dtype)
    pre = _draw_kv(seed, _PREFIX, [()], [prefix], hkv, d, 0.5, dtype)[0] if prefix else None
    kv = _draw_kv(seed, _KV, [(s,) for s in range(num_seqs)], [int(x) for x in priv], hkv, d, 0.5, dtype)
    T = 1 << 40
    ops = [("add", T)]
    if prefix:
        ops.append(("append", [(T, pre[0], pre[1])]))
    ops += [("fork", T, s) for s in range(num_seqs)]
    ops.append(("free", T))
    body = [(s, kv[s][0][:-1], kv[s][1][:-1]) for s in range(num_seqs) if priv[s] > 1]
    if body:
        ops.append(("append", body))
    ops.append(("append", [(s, kv[s][0][-1:], kv[s][1][-1:]) for s in range(num_seqs)]))
    return Workload(name="8b-gqa-prefix", dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    block_size=block_size, num_blocks=nb, free_order=free_order,
                    scale=float(np.float32(1.0 / math.sqrt(d))), partition_size=partition_size,
                    ops=ops, batch=list(range(num_seqs)), q=q, lmax=prefix + cap, value_scale=0.5,
                    notes={"prefix": prefix, "private": priv.tolist()})


def parallel_sampling(seed=3, prompts=8, n=4, prompt_len=512, max_extra=15, max_private=256,
                      hkv=40, d=128, block_size=16, dtype="f16", checks=None):
    """Parallel sampling with copy-on-write.

    Prompt p has prompt_len + s_p tokens, s_p ~ U{1..max_extra} (so its last block is partial
    and shared). Its n branches fork it; branch b then appends p_b ~ U{0..max_private} private
    tokens, one per decode step, all branches stepping together. ``checks`` lists the steps
    after which attention is evaluated (default: first, middle and last step).
    """
    r = _rng(seed, _LENGTHS)
    sp = r.integers(1 if max_extra > 0 else 0, max_extra + 1, size=prompts) if max_extra > 0 \
        else np.zeros(prompts, dtype=np.int64)
    pb = r.integers(0, max_private + 1, size=(prompts, n))
    L0 = prompt_len + sp
    bs = block_size
    need = 0
    for p in range(prompts):
        need += -(-int(L0[p]) // bs)
        for b in range(n):
            need += -(-int(L0[p] + pb[p, b]) // bs) - int(L0[p]) // bs
    nb = _pool_size(need)
    free_order = _rng(seed, _FREE).permutation(nb).astype(np.int32)
    S = prompts * n
    q = normal(_rng(seed, _Q), (S, hkv, d), 0.5, dtype)
    pk = _draw_kv(seed, _PROMPT, [(p,) for p in range(prompts)], [int(x) for x in L0], hkv, d, 0.5, dtype)
    bk = _draw_kv(seed, _KV, [(s,) for s in range(S)], [int(pb.flat[s]) for s in range(S)], hkv, d, 0.5, dtype)
    T0 = 1 << 40
    ops = []
    for p in range(prompts):
        ops += [("add", T0 + p), ("append", [(T0 + p, pk[p][0], pk[p][1])])]
    for p in range(prompts):
        ops += [("fork", T0 + p, p * n + b) for b in range(n)]
    ops += [("free", T0 + p) for p in range(prompts)]
    steps = int(pb.max(initial=0))
    if checks is None:
        checks = sorted({1, max(1, (steps + 1) // 2), steps}) if steps else []
    for i in range(steps):
        batch = [(s, bk[s][0][i:i + 1], bk[s][1][i:i + 1]) for s in range(S) if pb.flat[s] > i]
        ops.append(("append", batch))
        if (i + 1) in checks:
            ops.append(("check",))
    return Workload(name="cow-sampling", dtype=dtype, num_q_heads=hkv, num_kv_heads=hkv, head_dim=d,
                    block_size=bs, num_blocks=nb, free_order=free_order,
                    scale=float(np.float32(1.0 / math.sqrt(d))), partition_size=0, ops=ops,
                    batch=list(range(S)), q=q, lmax=int((L0[:, None] + pb).max()), value_scale=0.5,
                    notes={"s_p": sp.tolist(), "private": pb.tolist(), "steps": steps, "checks": checks})


def beam_search(seed=8, beams=4, fanout=3, steps=12, prompt_len=70, hq=8, hkv=8, d=128, block_size=16,
                dtype="f16"):
    """A beam-search schedule over one prompt, as seeded draws only: the prompt's K/V rows, and per
    step one score per candidate (each of the ``beams`` live beams forks ``fanout`` candidates, and the
    ``beams`` highest scores survive), the surviving beams' new K/V rows and their queries.

    The scores stand in for a model's sequence log-probabilities; which candidate survives is
    scheduling, not the method's arithmetic. A prompt whose length is not a multiple of the block
    size leaves a partly filled last block that every beam shares, so the first step copies it.
    """
    r = _rng(seed, _SCORES)
    pk = _draw_kv(seed, _PROMPT, [()], [prompt_len], hkv, d, 0.5, dtype)[0]
    sched = []
    live = 1  # the prompt's sequence
    for t in range(steps):
        keep = min(beams, live * fanout)
        kr = _rng(seed, _KV, t)
        sched.append({
            "scores": r.random(live * fanout),
            "k": normal(kr, (keep, hkv, d), 0.5, dtype),
            "v": normal(kr, (keep, hkv, d), 0.5, dtype),
            "q": normal(_rng(seed, _Q, t), (keep, hq, d), 0.5, dtype),
        })
        live = keep
    # blocks: the prompt's, plus at most one new block per surviving beam per step
    nb = _pool_size(-(-prompt_len // block_size) + beams * (steps + 1))
    free_order = _rng(seed, _FREE).permutation(nb).astype(np.int32)
    return {"prompt_k": pk[0], "prompt_v": pk[1], "steps": sched, "beams": beams, "fanout": fanout,
            "num_blocks": nb, "free_order": free_order, "block_size": block_size, "dtype": dtype,
            "hq": hq, "hkv": hkv, "d": d, "scale": float(np.float32(1.0 / math.sqrt(d)))}


def prefix_cache_requests(seed=6, system_lens=(69, 128, 200), requests=12, private=(1, 100), hq=16, hkv=8,
                          d=128, block_size=16, dtype="f16", vocab=32000):
    """Requests that open with one of a few shared system prompts (the lesson note, section
    3.1), each added with its whole prompt through the prefix cache, some freed as later ones
    arrive (so cached blocks are found again after falling free), then one decode step.

    A system prompt's token ids and its keys/values are drawn per (system prompt, position), so
    every request that opens with it carries the same rows there; the private part is drawn per
    request. Op ("prompt", sid, token_ids, k, v) adds a sequence with its whole prompt."""
    r = _rng(seed, _LENGTHS)
    kinds = r.integers(0, len(system_lens), size=requests)
    plen = r.integers(private[0], private[1] + 1, size=requests)
    sys_tok = [_rng(seed, _SYSTEM, s).integers(0, vocab, size=L).astype(np.int32) for s, L in enumerate(system_lens)]
    sys_kv = _draw_kv(seed, _SYSKV, [(s,) for s in range(len(system_lens))], list(system_lens), hkv, d, 0.5, dtype)
    prv_kv = _draw_kv(seed, _KV, [(i,) for i in range(requests)], [int(x) + 1 for x in plen], hkv, d, 0.5, dtype)
    ops, live = [], []
    for i in range(requests):
        s = int(kinds[i])
        toks = np.concatenate([sys_tok[s], _rng(seed, _TOKENS, i).integers(0, vocab, size=int(plen[i])).astype(np.int32)])
        k = np.concatenate([sys_kv[s][0], prv_kv[i][0][:-1]])
        v = np.concatenate([sys_kv[s][1], prv_kv[i][1][:-1]])
        ops.append(("prompt", i, toks, k, v))
        live.append(i)
        if i % 4 == 3:  # a request finishes: its blocks fall free, the hashed ones stay cached
            gone = live.pop(1)
            ops.append(("free", gone))
    ops.append(("append", [(i, prv_kv[i][0][-1:], prv_kv[i][1][-1:]) for i in live]))
    need = sum(-(-(system_lens[int(kinds[i])] + int(plen[i]) + 1) // block_size) for i in range(requests))
    nb = _pool_size(need)
    free_order = _rng(seed, _FREE).permutation(nb).astype(np.int32)
    q = normal(_rng(seed, _Q), (len(live), hq, d), 0.5, dtype)
    return Workload(name="prefix-cache", dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    block_size=block_size, num_blocks=nb, free_order=free_order,
                    scale=float(np.float32(1.0 / math.sqrt(d))), partition_size=0, ops=ops, batch=live, q=q,
                    lmax=int(max(system_lens) + private[1] + 1), value_scale=0.5,
                    notes={"kinds": kinds.tolist(), "private": plen.tolist()})


def serving_requests(seed=7, n=2000, prompt_median=160, output_median=200, sigma=1.0, max_context=2048,
                     rate=None):
    """Request lengths and arrival steps for the memory simulator: prompt and output lengths
    log-normal around the given medians, prompt + output within max_context (the reservation
    of the contiguous scheme, lesson note section 1), arrivals a Poisson process of `rate`
    requests per step (None: all at step 0). Returns int32 arrays (arrival, prompt, output)."""
    r = _rng(seed, _REQUESTS)
    prompt = np.clip(np.rint(r.lognormal(math.log(prompt_median), sigma, n)), 1, max_context - 1).astype(np.int64)
    output = np.clip(np.rint(r.lognormal(math.log(output_median), sigma, n)), 1, max_context - prompt).astype(np.int64)
    if rate is None:
        arrival = np.zeros(n, np.int64)
    else:
        arrival = np.floor(np.cumsum(r.exponential(1.0 / rate, n))).astype(np.int64)
    return arrival.astype(np.int32), prompt.astype(np.int32), output.astype(np.int32)


def kv_bytes_per_token(num_kv_heads, head_dim, elt_bytes):
    """Bytes of K plus V per token per layer: 2 * Hkv * d * e."""
    return 2 * num_kv_heads * head_dim * elt_bytes
