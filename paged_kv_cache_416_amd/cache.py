"""PagedKVCache: the native block pool plus one layer's device K/V caches, driven step by step.

Mirrors the pages' split of roles ("vLLM and PagedAttention" slide 16): the host side
owns the block tables and assigns slots; each step it ships slot numbers and tables to
the device, where copy_blocks, reshape_and_cache and the attention kernel run on one stream.
"""
from __future__ import annotations

import numpy as np
import torch

from . import kernels
from .pool import Pool

_POISON_BITS = {torch.float32: 0x7FC00000, torch.float16: 0x7E00, torch.bfloat16: 0x7FC0}
_INT_VIEW = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}


def poison_(t: torch.Tensor) -> torch.Tensor:
    """Fill a float tensor with quiet NaNs (a fill kernel, no memset), so stray reads show up."""
    t.view(_INT_VIEW[t.dtype]).fill_(_POISON_BITS[t.dtype])
    return t


class PagedKVCache:
    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, dtype, device=None, free_order=None,
                 poison=True):
        self.device = torch.device(device or "cuda")
        self.pool = Pool(num_blocks, block_size, free_order)
        self.block_size = block_size
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.dtype = dtype
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.k = torch.empty(shape, dtype=dtype, device=self.device)
        self.v = torch.empty(shape, dtype=dtype, device=self.device)
        if poison:
            poison_(self.k)
            poison_(self.v)
        self.last_slots = None
        self.last_pairs = None

    # -- scheduler side -------------------------------------------------
    def add(self, sid):
        self.pool.add(sid)

    def fork(self, parent, child):
        self.pool.fork(parent, child)

    def free(self, sid):
        self.pool.free(sid)

    def add_prompt(self, sid, tokens, keys, values):
        """Add sequence sid with its prompt through the prefix cache: keys/values [n, Hkv, D] device
        tensors for the whole prompt; rows of cached tokens are not written. Returns n_cached."""
        slots, n_cached = self.pool.add_prompt(sid, tokens)
        self.last_slots, self.last_pairs = slots, np.zeros((0, 2), np.int32)
        if len(slots) > n_cached:
            kernels.reshape_and_cache(keys, values, self.k, self.v, torch.from_numpy(slots).to(self.device))
        return n_cached

    def append(self, sids, keys, values):
        """Append keys[i]/values[i] ([n_i, Hkv, D] device tensors) to sequence sids[i], all or nothing.

        Runs copy-on-write copies first, then writes every new token into its slot, on one stream.
        """
        reqs = [(int(s), int(k.shape[0])) for s, k in zip(sids, keys)]
        slots, pairs = self.pool.append(reqs)
        self.last_slots, self.last_pairs = slots, pairs
        if len(pairs):
            kernels.copy_blocks([self.k], [self.v], pairs)
        if len(slots):
            key = torch.cat(list(keys)) if len(keys) > 1 else keys[0]
            val = torch.cat(list(values)) if len(values) > 1 else values[0]
            sm = torch.from_numpy(np.ascontiguousarray(slots)).to(self.device)
            kernels.reshape_and_cache(key, val, self.k, self.v, sm)
        return slots, pairs

    def tables(self, sids, pad=-1):
        """Device block tables, device lengths and the host bound on the lengths."""
        tb, ctx = self.pool.tables(sids, pad=pad)
        return (torch.from_numpy(tb).to(self.device), torch.from_numpy(ctx).to(self.device),
                int(ctx.max(initial=0)))

    # -- device side ----------------------------------------------------
    def shared_prefix_lens(self, sids):
        """Device int32 [n]: tokens of each sequence in its leading shared blocks (the cached-load hint)."""
        return torch.from_numpy(self.pool.shared_prefix_lens(sids)).to(self.device)

    def attention(self, q, sids, scale, partition_size=0, flags=0, out=None, cached_lens=None):
        """cached_lens: None, "shared" (from the pool's reference counts) or a device int32 [n]."""
        tb, ctx, mx = self.tables(sids)
        out = torch.empty_like(q) if out is None else out
        ws = kernels.alloc_workspace(q.shape[0], q.shape[1], q.shape[2], mx, partition_size, self.device)
        if isinstance(cached_lens, str):
            cached_lens = self.shared_prefix_lens(sids)
        return kernels.paged_attention_decode(out, q, self.k, self.v, tb, ctx, mx, scale, partition_size, ws, flags,
                                              cached_lens)


def to_device(a: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    """Upload a storage array (float32 / float16 / uint16 bf16 bits) as a tensor of `dtype`."""
    if dtype == torch.bfloat16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def run_ops(cache: PagedKVCache, ops, dtype, on_check=None):
    """Replay a list of scheduler operations:
    ("add", sid) | ("fork", parent, child) | ("free", sid) | ("append", [(sid, k, v), ...]) | ("check",)
    | ("prompt", sid, token_ids, k, v) (a sequence added with its whole prompt through the prefix cache).
    k, v are host storage arrays [n, Hkv, D]. on_check() is called at each ("check",)."""
    for op in ops:
        kind = op[0]
        if kind == "add":
            cache.add(op[1])
        elif kind == "fork":
            cache.fork(op[1], op[2])
        elif kind == "free":
            cache.free(op[1])
        elif kind == "append":
            sids = [sid for sid, _, _ in op[1]]
            keys = to_device(np.concatenate([k for _, k, _ in op[1]]), dtype, cache.device)
            vals = to_device(np.concatenate([v for _, _, v in op[1]]), dtype, cache.device)
            # one launch per step: split back into per-sequence views only for the row counts
            counts = [k.shape[0] for _, k, _ in op[1]]
            ks = list(torch.split(keys, counts))
            vs = list(torch.split(vals, counts))
            cache.append(sids, ks, vs)
        elif kind == "prompt":
            cache.add_prompt(op[1], op[2], to_device(op[3], dtype, cache.device), to_device(op[4], dtype, cache.device))
        elif kind == "check":
            if on_check is not None:
                on_check()
        else:
            raise ValueError(f"unknown op {kind}")
