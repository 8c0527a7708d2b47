"""Python handle on the native host block-pool allocator (pkv_pool_* / pkv_seq_* in include/pkv.h)."""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import PKV_ENOMEM, PkvError, check, load

_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)


def _i32p(a):
    return a.ctypes.data_as(_pi32)


def _i64p(a):
    return a.ctypes.data_as(_pi64)


class OutOfBlocks(PkvError):
    pass


class Pool:
    """A pool of fixed-size physical blocks with per-sequence block tables (host state)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._lib = load()
        h = ctypes.c_void_p()
        fo = None
        if free_order is not None:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            if fo.shape != (num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
        check(self._lib.pkv_pool_create(num_blocks, block_size, _i32p(fo) if fo is not None else None,
                                        ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_pool_destroy(h)
            self._h = None

    # queries
    def num_free(self) -> int:
        return int(self._lib.pkv_pool_num_free(self._h))

    def ref_count(self, block: int) -> int:
        return int(self._lib.pkv_block_ref_count(self._h, block))

    def length(self, sid: int) -> int:
        n = int(self._lib.pkv_seq_len(self._h, sid))
        if n < 0:
            check(n)
        return n

    def blocks(self, sid: int):
        nb = int(self._lib.pkv_seq_num_blocks(self._h, sid))
        if nb < 0:
            check(nb)
        out = np.zeros(max(nb, 1), np.int32)
        n = int(self._lib.pkv_seq_blocks(self._h, sid, _i32p(out), nb))
        if n < 0:
            check(n)
        return out[:n].tolist()

    # lifecycle
    def add(self, sid: int):
        check(self._lib.pkv_seq_add(self._h, sid))

    def free(self, sid: int):
        check(self._lib.pkv_seq_free(self._h, sid))

    def fork(self, parent: int, child: int):
        check(self._lib.pkv_seq_fork(self._h, parent, child))

    def append(self, requests):
        """requests: [(sid, n_tokens), ...] -> (slots int64 [sum n], pairs int32 [P, 2]); all or nothing."""
        ids = np.ascontiguousarray([r[0] for r in requests], dtype=np.int64)
        ns = np.ascontiguousarray([r[1] for r in requests], dtype=np.int32)
        total = int(ns.sum()) if len(ns) else 0
        slots = np.zeros(max(total, 1), np.int64)
        max_pairs = len(requests)
        pairs = np.zeros(2 * max(max_pairs, 1), np.int32)
        npairs = ctypes.c_int32(0)
        rc = self._lib.pkv_seq_append(self._h, _i64p(ids), _i32p(ns), len(requests), _i64p(slots), _i32p(pairs),
                                      max_pairs, ctypes.byref(npairs))
        if rc == PKV_ENOMEM:
            raise OutOfBlocks(rc, self._lib.pkv_last_error().decode())
        check(rc)
        return slots[:total], pairs[:2 * npairs.value].reshape(-1, 2)

    def tables(self, sids, max_blocks=None, pad=-1):
        """Dense block tables int32 [n, max_blocks] (padded) and lengths int32 [n], host arrays."""
        ids = np.ascontiguousarray(sids, dtype=np.int64)
        if max_blocks is None:
            max_blocks = max([len(self.blocks(int(s))) for s in ids] + [1])
        tb = np.zeros((len(ids), max_blocks), np.int32)
        ctx = np.zeros(len(ids), np.int32)
        check(self._lib.pkv_build_block_tables(self._h, _i64p(ids), len(ids), max_blocks, pad, _i32p(tb),
                                               _i32p(ctx)))
        return tb, ctx

    def shared_prefix_lens(self, sids):
        """Tokens of each sequence in its leading shared blocks (count above one), int32 [n], host."""
        ids = np.ascontiguousarray(sids, dtype=np.int64)
        out = np.zeros(len(ids), np.int32)
        check(self._lib.pkv_shared_prefix_lens(self._h, _i64p(ids), len(ids), _i32p(out)))
        return out

    def migrate(self, dst: "Pool", sids):
        """Move sequences sids to pool dst, all or nothing -> (src block, dst block) pairs int32 [P, 2]
        to copy (preemption by swap and its recovery)."""
        ids = np.ascontiguousarray(sids, dtype=np.int64)
        max_pairs = sum(len(self.blocks(int(s))) for s in ids) if all(self._has(int(s)) for s in ids) else 0
        pairs = np.zeros(2 * max(max_pairs, 1), np.int32)
        npairs = ctypes.c_int32(0)
        rc = self._lib.pkv_seq_migrate(self._h, dst._h, _i64p(ids), len(ids), _i32p(pairs), max_pairs,
                                       ctypes.byref(npairs))
        if rc == PKV_ENOMEM:
            raise OutOfBlocks(rc, self._lib.pkv_last_error().decode())
        check(rc)
        return pairs[:2 * npairs.value].reshape(-1, 2)

    def _has(self, sid: int) -> bool:
        return self._lib.pkv_seq_len(self._h, sid) >= 0

    def add_prompt(self, sid: int, tokens):
        """Add sequence sid with prompt token ids (prefix cache) -> (slots int64 [n], n_cached):
        slots of cached tokens are -1."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.zeros(max(len(toks), 1), np.int64)
        n_cached = ctypes.c_int32(0)
        rc = self._lib.pkv_seq_add_prompt(self._h, sid, _i32p(toks), len(toks), _i64p(slots), ctypes.byref(n_cached))
        if rc == PKV_ENOMEM:
            raise OutOfBlocks(rc, self._lib.pkv_last_error().decode())
        check(rc)
        return slots[:len(toks)], n_cached.value

    def num_cached(self) -> int:
        return self._lib.pkv_pool_num_cached(self._h)


def prompt_digests(tokens, block_size):
    """Chained SHA-256 digests of the full blocks of a token stream -> bytes array [k, 32]."""
    toks = np.ascontiguousarray(tokens, dtype=np.int32)
    k = len(toks) // block_size
    out = np.zeros((max(k, 1), 32), np.uint8)
    n = load().pkv_prompt_digests(_i32p(toks), len(toks), block_size,
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), k)
    check(0 if n >= 0 else n)
    return out[:n]
