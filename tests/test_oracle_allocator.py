"""Pins of the oracle's allocator model: invariants the pages state, checked after every operation."""
import numpy as np
import pytest
from hypothesis import settings, strategies as st
from hypothesis.stateful import RuleBasedStateMachine, initialize, invariant, precondition, rule

from oracle.allocator import BlockPool, OutOfBlocks


def test_free_order_is_pop_order():
    pool = BlockPool(5, 4, [3, 0, 4, 1, 2])
    pool.add(0)
    pool.append([(0, 20)])
    assert pool.blocks(0) == [3, 0, 4, 1, 2]


def test_freed_blocks_reused_last_block_first():
    pool = BlockPool(6, 4)
    pool.add(0)
    pool.append([(0, 9)])  # blocks 0, 1, 2
    pool.free_seq(0)
    pool.add(1)
    pool.append([(1, 4)])
    assert pool.blocks(1) == [2]


def test_cow_copies_n_minus_1_times():
    """n branches sharing a partial last block: n-1 copies; the last writer writes in place."""
    for n in (2, 4, 7):
        pool = BlockPool(64, 16)
        pool.add("p")
        pool.append([("p", 37)])
        for b in range(n):
            pool.fork("p", b)
        pool.free_seq("p")
        last = pool.blocks(0)[-1]
        assert pool.ref[last] == n
        slots, pairs = pool.append([(b, 1) for b in range(n)])
        assert len(pairs) == n - 1
        assert all(src == last for src, _ in pairs)
        assert pool.blocks(n - 1)[-1] == last and pool.ref[last] == 1
        # only the last block was ever copied: the full blocks are still shared by all
        for j in range(2):
            assert pool.ref[pool.blocks(0)[j]] == n
        pool.check_invariants()
        # the token goes to the copied block, in the same offset
        for b in range(n):
            assert slots[b] == pool.blocks(b)[-1] * 16 + 37 % 16


def test_cow_not_needed_when_shared_block_is_full():
    pool = BlockPool(16, 16)
    pool.add(0)
    pool.append([(0, 32)])
    pool.fork(0, 1)
    _, pairs = pool.append([(0, 1), (1, 1)])
    assert pairs == []
    assert pool.ref[pool.blocks(0)[0]] == 2 and pool.ref[pool.blocks(0)[1]] == 2
    pool.check_invariants()


def test_out_of_blocks_changes_nothing():
    pool = BlockPool(4, 4)
    pool.add(0)
    pool.add(1)
    pool.append([(0, 6)])
    snap = (list(pool.free), list(pool.ref), {k: (list(v[0]), v[1]) for k, v in pool.seqs.items()})
    with pytest.raises(OutOfBlocks):
        pool.append([(1, 4), (0, 7)])  # 1 + 2 blocks wanted, 2 free
    assert (pool.free, pool.ref, {k: (v[0], v[1]) for k, v in pool.seqs.items()}) == snap


def test_waste_bounded_by_last_block():
    """Only the last block can be partly empty: allocated slots - length < B for an unshared sequence."""
    rng = np.random.default_rng(0)
    pool = BlockPool(4096, 16, rng.permutation(4096))
    for s in range(50):
        pool.add(s)
        n = int(rng.integers(0, 300))
        pool.append([(s, n)])
        assert 0 <= len(pool.blocks(s)) * 16 - pool.length(s) <= 15


class PoolMachine(RuleBasedStateMachine):
    """Random add / append / fork / free sequences; the pool's invariants hold after every step."""

    @initialize(N=st.integers(1, 24), B=st.sampled_from([1, 2, 4, 16]), seed=st.integers(0, 1000))
    def setup(self, N, B, seed):
        self.pool = BlockPool(N, B, np.random.default_rng(seed).permutation(N))
        self.next_id = 0
        self.tokens = {}  # sid -> list of token ids written, in order (logical contents)
        self.slot_owner = {}  # slot -> token id currently stored

    @rule()
    def add(self):
        self.pool.add(self.next_id)
        self.tokens[self.next_id] = []
        self.next_id += 1

    @precondition(lambda self: self.tokens)
    @rule(data=st.data())
    def fork(self, data):
        p = data.draw(st.sampled_from(sorted(self.tokens)))
        self.pool.fork(p, self.next_id)
        self.tokens[self.next_id] = list(self.tokens[p])
        self.next_id += 1

    @precondition(lambda self: self.tokens)
    @rule(data=st.data())
    def free(self, data):
        s = data.draw(st.sampled_from(sorted(self.tokens)))
        self.pool.free_seq(s)
        del self.tokens[s]

    @precondition(lambda self: self.tokens)
    @rule(data=st.data())
    def append(self, data):
        sids = data.draw(st.lists(st.sampled_from(sorted(self.tokens)), min_size=1, max_size=4, unique=True))
        ns = [data.draw(st.integers(0, 9)) for _ in sids]
        free_before = self.pool.num_free()
        try:
            slots, pairs = self.pool.append(list(zip(sids, ns)))
        except OutOfBlocks:
            assert self.pool.num_free() == free_before
            return
        B = self.pool.block_size
        # copy pairs: the copy carries the old block's contents (as a block copy does)
        for src, dst in pairs:
            for o in range(B):
                if src * B + o in self.slot_owner:
                    self.slot_owner[dst * B + o] = self.slot_owner[src * B + o]
        i = 0
        for sid, n in zip(sids, ns):
            for _ in range(n):
                tok = (sid, len(self.tokens[sid]))
                self.tokens[sid].append(tok)
                self.slot_owner[slots[i]] = tok
                i += 1
        assert i == len(slots)

    @invariant()
    def pool_invariants(self):
        if hasattr(self, "pool"):
            self.pool.check_invariants()

    @invariant()
    def every_sequence_reads_its_own_tokens(self):
        """Through its table, each sequence sees exactly the tokens written for it, in order."""
        if not hasattr(self, "pool"):
            return
        B = self.pool.block_size
        for sid, toks in self.tokens.items():
            blocks = self.pool.blocks(sid)
            assert self.pool.length(sid) == len(toks)
            for t, tok in enumerate(toks):
                slot = blocks[t // B] * B + t % B
                owner = self.slot_owner.get(slot)
                # a forked child sees the parent's token ids for the shared prefix
                assert owner is not None
                assert owner[1] == tok[1]


PoolMachine.TestCase.settings = settings(max_examples=120, stateful_step_count=40, deadline=None)
TestPoolMachine = PoolMachine.TestCase
