"""Reference model of the block-pool allocator -- TEST INFRASTRUCTURE ONLY (pure Python).

Follows the pages' statement of the problem:
  * one pool of fixed-size physical blocks, and a request may take whichever
    block is free ("vLLM and PagedAttention" slides, slide 12, and the "Week 22
    Day 2" lesson note, section 2);
  * a per-sequence block table maps logical block j (tokens j*B .. j*B+B-1) to
    a physical block (slide 10; lesson note section 2, block-table diagram);
  * a new block is taken only when the last one is full (slide 11);
  * sharing increments a block's reference count (lesson note section 3.1);
  * a sequence about to write into a shared, partly filled last block gets a
    private copy first, and no other block is ever duplicated (slide 13, lesson
    note section 3.2);
  * finished sequences return their blocks at once (lesson note section 4);
  * a request that cannot get all its blocks gets none (slide 15).

Readings where the pages fix no detail (the GPU library's allocator makes the
same choices independently):
  * free blocks form a LIFO stack; ``free_order[0]`` is handed out first;
  * a freed sequence returns its blocks in logical order, so its last block is
    the next one handed out;
  * within one batched append, sequences are served in the order given, and
    the whole batch fails, changing nothing, if the pool runs short.

Prefix cache (lesson note section 3.1: prompt blocks are looked up by a
cryptographic digest; a new request whose block has the digest of a held block
maps that block and increments its count). Readings: the digest of full prompt block j is SHA-256 (Python's hashlib)
of the previous block's digest (32 zero bytes for the first) followed by the
block's token ids as little-endian int32, so equal digests mean equal prefixes;
only full prompt blocks are hashed and hits are taken as a prefix of the prompt; a
hashed block that falls free keeps its digest until the pool needs it -- free
blocks without a digest are handed out first (the LIFO stack above), then hashed
free blocks, least recently freed first, each losing its digest. A digest is held by one
block: when a new prompt block's digest is already held (a later block of a chain whose
earlier block was evicted), the new block takes it over and the old block becomes an
ordinary block, joining the LIFO stack if it is free.
"""
from __future__ import annotations

import copy
import hashlib

import numpy as np


def prompt_digests(tokens, block_size):
    """Chained digests of the full blocks of a token stream (lesson note section 3.1)."""
    out, prev = [], bytes(32)
    for j in range(len(tokens) // block_size):
        block = np.asarray(tokens[j * block_size:(j + 1) * block_size], dtype="<i4").tobytes()
        prev = hashlib.sha256(prev + block).digest()
        out.append(prev)
    return out


class OutOfBlocks(Exception):
    pass


class BlockPool:
    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = order[::-1]  # top of the stack is the end of the list
        self.cached_free = []  # free blocks that keep a digest, least recently freed first
        self.digest_of = {}  # block -> digest
        self.block_of = {}  # digest -> block
        self.ref = [0] * num_blocks
        self.seqs = {}  # sid -> [blocks(list), length(int)]

    # -- queries ---------------------------------------------------------
    def num_free(self):
        return len(self.free) + len(self.cached_free)

    def num_cached(self):
        return len(self.block_of)

    def length(self, sid):
        return self.seqs[sid][1]

    def blocks(self, sid):
        return list(self.seqs[sid][0])

    # -- lifecycle -------------------------------------------------------
    def add(self, sid):
        if sid in self.seqs:
            raise KeyError(f"sequence {sid} exists")
        self.seqs[sid] = [[], 0]

    def fork(self, parent, child):
        if child in self.seqs:
            raise KeyError(f"sequence {child} exists")
        blocks, n = self.seqs[parent]
        for b in blocks:
            self.ref[b] += 1
        self.seqs[child] = [list(blocks), n]

    def free_seq(self, sid):
        blocks, _ = self.seqs.pop(sid)
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self._release(b)

    def _release(self, b):
        if b in self.digest_of:
            self.cached_free.append(b)
        else:
            self.free.append(b)

    def _take(self):
        if self.free:
            b = self.free.pop()
        else:
            b = self.cached_free.pop(0)
            del self.block_of[self.digest_of.pop(b)]
        self.ref[b] = 1
        return b

    def add_prompt(self, sid, tokens):
        """New sequence with a prompt (prefix cache). Returns (slots, n_cached): -1 for the leading
        tokens whose blocks were found by digest, the slot of every other token."""
        if sid in self.seqs:
            raise KeyError(f"sequence {sid} exists")
        B = self.block_size
        digests = prompt_digests(tokens, B)
        hits = []
        for d in digests:
            if d not in self.block_of:
                break
            hits.append(self.block_of[d])
        revive = sum(1 for b in hits if self.ref[b] == 0)
        fresh = len(digests) - len(hits) + (1 if len(tokens) % B else 0)
        if revive + fresh > self.num_free():
            raise OutOfBlocks()
        blocks = []
        for b in hits:
            if self.ref[b] == 0:
                self.cached_free.remove(b)
            self.ref[b] += 1
            blocks.append(b)
        for d in digests[len(hits):]:
            b = self._take()
            old = self.block_of.get(d)
            if old is not None:
                # a later block of a chain whose earlier block was evicted: the new block takes
                # the digest over and the old one becomes an ordinary block (free, if unused)
                del self.digest_of[old]
                if self.ref[old] == 0:
                    self.cached_free.remove(old)
                    self.free.append(old)
            self.digest_of[b] = d
            self.block_of[d] = b
            blocks.append(b)
        if len(tokens) % B:
            blocks.append(self._take())
        self.seqs[sid] = [blocks, len(tokens)]
        n_cached = len(hits) * B
        slots = [-1 if t < n_cached else blocks[t // B] * B + t % B for t in range(len(tokens))]
        return slots, n_cached

    def _append_one(self, sid, n):
        B = self.block_size
        blocks, length = self.seqs[sid]
        pairs = []
        if n == 0:
            return [], pairs
        if length % B and self.ref[blocks[-1]] > 1:
            if self.num_free() == 0:
                raise OutOfBlocks()
            old = blocks[-1]
            new = self._take()
            self.ref[old] -= 1
            blocks[-1] = new
            pairs.append((old, new))
        while len(blocks) * B < length + n:
            if self.num_free() == 0:
                raise OutOfBlocks()
            blocks.append(self._take())
        slots = [blocks[t // B] * B + t % B for t in range(length, length + n)]
        self.seqs[sid][1] = length + n
        return slots, pairs

    def append(self, requests):
        """requests: [(sid, n_tokens), ...]. Returns (slots, copy pairs); all or nothing."""
        sids = [s for s, _ in requests]
        if len(set(sids)) != len(sids):
            raise ValueError("a sequence appears twice in one batch")
        for s in sids:
            if s not in self.seqs:
                raise KeyError(f"unknown sequence {s}")
        saved = (list(self.free), list(self.ref), copy.deepcopy(self.seqs), list(self.cached_free),
                 dict(self.digest_of), dict(self.block_of))
        slots, pairs = [], []
        try:
            for sid, n in requests:
                sl, pr = self._append_one(sid, int(n))
                slots += sl
                pairs += pr
        except OutOfBlocks:
            self.free, self.ref, self.seqs, self.cached_free, self.digest_of, self.block_of = saved
            raise
        return slots, pairs

    def migrate_to(self, dst, sids):
        """Move whole sequences to another pool (preemption by swap, and its recovery: slide 15 of
        the "vLLM and PagedAttention" deck -- a request leaves all at once and comes back by
        swap). Returns the (block here, block in dst) pairs whose contents must be copied.

        Readings (the pages say only "swap"): each distinct block the moving sequences map is
        copied once, into a fresh dst block taken in first-use order (sequence order, then
        logical order), so blocks they share stay shared in dst with the same number of
        sharers; the sequences then leave this pool exactly as free_seq would, in the order
        given, so a block another (unmoved) sequence still maps stays here. All or nothing: a
        dst pool too short to take every block changes neither pool."""
        if dst is self or dst.block_size != self.block_size:
            raise ValueError("migrate needs two pools of one block size")
        if len(set(sids)) != len(sids):
            raise ValueError("a sequence appears twice")
        for s in sids:
            if s not in self.seqs:
                raise KeyError(f"unknown sequence {s}")
            if s in dst.seqs:
                raise KeyError(f"sequence {s} exists in dst")
        sharers = {}
        first_use = []
        for s in sids:
            for b in self.seqs[s][0]:
                if b not in sharers:
                    sharers[b] = 0
                    first_use.append(b)
                sharers[b] += 1
        if len(first_use) > dst.num_free():
            raise OutOfBlocks()
        moved_to = {}
        for b in first_use:
            nb = dst._take()
            dst.ref[nb] = sharers[b]
            moved_to[b] = nb
        for s in sids:
            blocks, n = self.seqs[s]
            dst.seqs[s] = [[moved_to[b] for b in blocks], n]
            self.free_seq(s)
        return [(b, moved_to[b]) for b in first_use]

    def shared_prefix_len(self, sid):
        """Tokens of sid in the leading run of its blocks whose reference count is above one
        (blocks other sequences also hold; lesson note section 3.1, slide 14)."""
        blocks, n = self.seqs[sid]
        j = 0
        while j < len(blocks) and self.ref[blocks[j]] > 1:
            j += 1
        return min(n, j * self.block_size)

    def tables(self, sids, max_blocks, pad=-1):
        rows, ctx = [], []
        for s in sids:
            blocks, n = self.seqs[s]
            if len(blocks) > max_blocks:
                raise ValueError("max_blocks too small")
            rows.append(list(blocks) + [pad] * (max_blocks - len(blocks)))
            ctx.append(n)
        return rows, ctx

    def check_invariants(self):
        """One pool; reference counts count sharers; a block is free iff its count is zero; the
        digest index and the hashed free blocks agree."""
        N = self.num_blocks
        free = self.free + self.cached_free
        assert len(set(free)) == len(free)
        used = {b for blocks, _ in self.seqs.values() for b in blocks}
        assert len(free) + len(used) == N
        for b in range(N):
            holders = sum(blocks.count(b) for blocks, _ in self.seqs.values())
            assert self.ref[b] == holders, (b, self.ref[b], holders)
            assert (b in free) == (holders == 0)
        assert all(b in self.digest_of for b in self.cached_free) and not set(self.free) & set(self.digest_of)
        assert {d: b for b, d in self.digest_of.items()} == self.block_of
        B = self.block_size
        for blocks, n in self.seqs.values():
            assert len(blocks) == -(-n // B)
