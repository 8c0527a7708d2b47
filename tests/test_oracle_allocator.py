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


def test_shared_prefix_len_worked_example():
    """Shared prefix from the counts, worked by hand: a 42-token sequence (blocks of 16: two full,
    one holding 10) forked once shares all 42 tokens; the child's first append copies the shared
    partial block (slide 13), after which both sequences share exactly the two full blocks."""
    pool = BlockPool(16, 16)
    pool.add(0)
    pool.append([(0, 42)])
    assert pool.shared_prefix_len(0) == 0  # nothing shared yet
    pool.fork(0, 1)
    assert pool.shared_prefix_len(0) == 42 and pool.shared_prefix_len(1) == 42
    _, pairs = pool.append([(1, 1)])
    assert len(pairs) == 1
    assert pool.shared_prefix_len(0) == 32 and pool.shared_prefix_len(1) == 32
    pool.append([(0, 30)])  # private tokens past the shared blocks
    assert pool.shared_prefix_len(0) == 32 and pool.length(0) == 72
    pool.fork(1, 2)  # sequence 1's third block (private until now) becomes shared too
    assert pool.shared_prefix_len(1) == 43 and pool.shared_prefix_len(2) == 43
    assert pool.shared_prefix_len(0) == 32
    pool.free_seq(1)
    pool.free_seq(2)
    assert pool.shared_prefix_len(0) == 0
    pool.check_invariants()


def test_shared_prefix_len_stops_at_first_private_block():
    """Blocks shared after a private one do not count: the hint is a prefix of the table."""
    pool = BlockPool(8, 4)
    pool.add("a")
    pool.append([("a", 12)])
    pool.fork("a", "b")
    pool.append([("b", 4)])  # b: three shared full blocks + one private block
    assert pool.shared_prefix_len("b") == 12 and pool.shared_prefix_len("a") == 12
    pool.free_seq("a")
    assert pool.shared_prefix_len("b") == 0


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


class TwoPoolMachine(RuleBasedStateMachine):
    """A device pool and a host pool (slide 15: a preempted request leaves by swap and comes
    back): sequences move between them with migrate_to while add / fork / append / free go on.
    Pins the move without restating it: both pools' invariants after every step, every
    sequence still reads its own tokens through its table in the pool that holds it (block
    contents carried by the returned pairs, as a block copy carries them), the moved
    sequences map as many distinct blocks after the move as before (sharing kept), and a
    move the destination cannot take changes neither pool."""

    @initialize(nd=st.integers(1, 20), nh=st.integers(1, 20), B=st.sampled_from([1, 2, 4, 16]),
                seed=st.integers(0, 1000))
    def setup(self, nd, nh, B, seed):
        rng = np.random.default_rng(seed)
        self.pools = {"dev": BlockPool(nd, B, rng.permutation(nd)), "host": BlockPool(nh, B, rng.permutation(nh))}
        self.where = {}  # sid -> "dev" | "host"
        self.tokens = {}
        self.owner = {"dev": {}, "host": {}}  # pool -> slot -> token id
        self.next_id = 0

    def _ids(self, place):
        return sorted(s for s, w in self.where.items() if w == place)

    @rule()
    def add(self):
        self.pools["dev"].add(self.next_id)
        self.where[self.next_id] = "dev"
        self.tokens[self.next_id] = []
        self.next_id += 1

    @precondition(lambda self: self.where)
    @rule(data=st.data())
    def fork(self, data):
        p = data.draw(st.sampled_from(sorted(self.where)))
        self.pools[self.where[p]].fork(p, self.next_id)
        self.where[self.next_id] = self.where[p]
        self.tokens[self.next_id] = list(self.tokens[p])
        self.next_id += 1

    @precondition(lambda self: self.where)
    @rule(data=st.data())
    def free(self, data):
        s = data.draw(st.sampled_from(sorted(self.where)))
        self.pools[self.where.pop(s)].free_seq(s)
        del self.tokens[s]

    @precondition(lambda self: any(w == "dev" for w in self.where.values()))
    @rule(data=st.data())
    def append(self, data):
        pool = self.pools["dev"]
        sids = data.draw(st.lists(st.sampled_from(self._ids("dev")), min_size=1, max_size=3, unique=True))
        ns = [data.draw(st.integers(0, 9)) for _ in sids]
        try:
            slots, pairs = pool.append(list(zip(sids, ns)))
        except OutOfBlocks:
            return
        B, own = pool.block_size, self.owner["dev"]
        for src, dst in pairs:
            for o in range(B):
                if src * B + o in own:
                    own[dst * B + o] = own[src * B + o]
        i = 0
        for sid, n in zip(sids, ns):
            for _ in range(n):
                tok = (sid, len(self.tokens[sid]))
                self.tokens[sid].append(tok)
                own[slots[i]] = tok
                i += 1

    def _move(self, data, frm, to):
        sids = data.draw(st.lists(st.sampled_from(self._ids(frm)), min_size=1, max_size=4, unique=True))
        src, dst = self.pools[frm], self.pools[to]
        before = (list(src.free), list(src.ref), list(dst.free), list(dst.ref),
                  {s: src.blocks(s) for s in src.seqs})
        distinct = len({b for s in sids for b in src.blocks(s)})
        try:
            pairs = src.migrate_to(dst, sids)
        except OutOfBlocks:
            assert (list(src.free), list(src.ref), list(dst.free), list(dst.ref)) == before[:4]
            assert {s: src.blocks(s) for s in src.seqs} == before[4]
            assert distinct > dst.num_free()
            return
        assert len(pairs) == distinct == len({b for s in sids for b in dst.blocks(s)})
        B = src.block_size
        for a, b in pairs:  # the copy the caller runs
            for o in range(B):
                if a * B + o in self.owner[frm]:
                    self.owner[to][b * B + o] = self.owner[frm][a * B + o]
        for s in sids:
            self.where[s] = to

    @precondition(lambda self: any(w == "dev" for w in self.where.values()))
    @rule(data=st.data())
    def swap_out(self, data):
        self._move(data, "dev", "host")

    @precondition(lambda self: any(w == "host" for w in self.where.values()))
    @rule(data=st.data())
    def swap_in(self, data):
        self._move(data, "host", "dev")

    @invariant()
    def both_pools_consistent_and_every_sequence_reads_its_tokens(self):
        if not hasattr(self, "pools"):
            return
        for p in self.pools.values():
            p.check_invariants()
        for sid, toks in self.tokens.items():
            place = self.where[sid]
            pool, own = self.pools[place], self.owner[place]
            assert sid in pool.seqs and all(sid not in q.seqs for n, q in self.pools.items() if n != place)
            B = pool.block_size
            blocks = pool.blocks(sid)
            assert pool.length(sid) == len(toks)
            for t, tok in enumerate(toks):
                got = own.get(blocks[t // B] * B + t % B)
                assert got is not None and got[1] == tok[1]


TwoPoolMachine.TestCase.settings = settings(max_examples=120, stateful_step_count=40, deadline=None)
TestTwoPoolMachine = TwoPoolMachine.TestCase


def test_migrate_single_unshared_sequence_is_a_block_list_copy():
    """A lone unshared sequence moves to the next free blocks of dst in LIFO order, one pair per
    block in logical order, and its source blocks return to the free stack."""
    src, dst = BlockPool(8, 4, [5, 1, 6, 0, 2, 3, 4, 7]), BlockPool(6, 4, [3, 0, 5, 1, 2, 4])
    src.add(9)
    src.append([(9, 10)])  # blocks 5, 1, 6
    pairs = src.migrate_to(dst, [9])
    assert pairs == [(5, 3), (1, 0), (6, 5)]
    assert dst.blocks(9) == [3, 0, 5] and dst.length(9) == 10
    assert src.num_free() == 8 and src.free[-3:] == [5, 1, 6]


# ---------------------------------------------------------------- prefix cache (lesson note 3.1)

from oracle.allocator import prompt_digests  # noqa: E402


@pytest.mark.parametrize("B", [1, 7, 8, 16, 32])
def test_digests_chain_over_the_prefix(B):
    """Equal prompts give equal digests; changing one token of block j changes the digests of
    blocks j.. and of no earlier block (a block's digest stands for its whole prefix)."""
    rng = np.random.default_rng(B)
    toks = rng.integers(0, 50000, size=5 * B + 3 % B).tolist()
    d = prompt_digests(toks, B)
    assert len(d) == 5 and len(set(d)) == 5 and all(len(x) == 32 for x in d)
    assert prompt_digests(list(toks), B) == d
    for j in range(5):
        t2 = list(toks)
        t2[j * B + B // 2] += 1
        d2 = prompt_digests(t2, B)
        assert d2[:j] == d[:j] and all(a != b for a, b in zip(d2[j:], d[j:]))
    # the same block contents after a different prefix hash differently
    assert prompt_digests(toks[B:2 * B], B)[0] != d[1]


def test_shared_system_prompt_maps_the_same_blocks():
    p = BlockPool(16, 4)
    sys_prompt = [11, 12, 13, 14, 21, 22, 23, 24, 31, 32, 33, 34]
    s1, c1 = p.add_prompt(1, sys_prompt + [7, 8])
    assert c1 == 0 and -1 not in s1
    s2, c2 = p.add_prompt(2, sys_prompt + [9])
    assert c2 == 12 and s2[:12] == [-1] * 12 and s2[12] >= 0
    assert p.blocks(2)[:3] == p.blocks(1)[:3] and p.blocks(2)[3] != p.blocks(1)[3]
    assert [p.ref[b] for b in p.blocks(1)[:3]] == [2, 2, 2] and p.num_cached() == 3
    # a prompt that leaves the system prompt inside block 1 shares block 0 only
    s3, c3 = p.add_prompt(3, sys_prompt[:5] + [99] + sys_prompt[6:])
    assert c3 == 4 and p.blocks(3)[0] == p.blocks(1)[0] and p.blocks(3)[1] != p.blocks(1)[1]
    p.check_invariants()


def test_freed_prompt_blocks_stay_cached_until_needed():
    """Freed hashed blocks are found again; blocks without a digest are handed out before them,
    and then the least recently freed hashed block goes first."""
    p = BlockPool(6, 2)
    p.add_prompt(1, [1, 2, 3, 4])   # hashed blocks a, b
    p.add_prompt(2, [5, 6, 7])      # hashed c, partial d
    a, b = p.blocks(1)
    c, d = p.blocks(2)
    p.free_seq(1)
    p.free_seq(2)
    assert p.num_free() == 6 and p.num_cached() == 3
    _, n = p.add_prompt(3, [1, 2, 3, 4, 9])  # a and b revived, one new block for the tail
    assert n == 4 and p.blocks(3)[:2] == [a, b] and p.blocks(3)[2] not in (a, b, c)
    p.free_seq(3)  # a, b freed again (after c)
    p.add(4)
    p.append([(4, 8)])  # 4 blocks: the three unhashed free blocks first, then c (least recently freed)
    assert c not in p.blocks(4)[:3] and p.blocks(4)[3] == c and p.num_cached() == 2
    p.check_invariants()


def test_prompt_that_does_not_fit_changes_nothing():
    p = BlockPool(3, 4)
    p.add_prompt(1, list(range(8)))
    before = (list(p.free), list(p.cached_free), list(p.ref), dict(p.block_of))
    with pytest.raises(OutOfBlocks):
        p.add_prompt(2, list(range(100, 112)))
    assert (list(p.free), list(p.cached_free), list(p.ref), dict(p.block_of)) == before and 2 not in p.seqs


class PrefixCacheMachine(RuleBasedStateMachine):
    """Prompts built from a few shared system prompts and private suffixes; add_prompt / free /
    fork / append in any order. The cache tokens are not written (slot -1), so the check that
    every sequence reads its own token ids through its table proves each hit mapped a block
    holding exactly those tokens."""

    @initialize(N=st.integers(2, 24), B=st.sampled_from([1, 2, 4, 8]), seed=st.integers(0, 1000))
    def setup(self, N, B, seed):
        rng = np.random.default_rng(seed)
        self.pool = BlockPool(N, B, rng.permutation(N))
        self.systems = [rng.integers(0, 5, size=rng.integers(0, 3 * B + 2)).tolist() for _ in range(3)]
        self.toks = {}
        self.content = {}  # slot -> token id
        self.next = 0

    @rule(data=st.data())
    def add_prompt(self, data):
        base = data.draw(st.sampled_from(self.systems))
        tail = data.draw(st.lists(st.integers(0, 5), max_size=2 * self.pool.block_size))
        prompt = base + tail
        try:
            slots, n_cached = self.pool.add_prompt(self.next, prompt)
        except OutOfBlocks:
            return
        assert all(s == -1 for s in slots[:n_cached]) and all(s >= 0 for s in slots[n_cached:])
        for s, t in zip(slots, prompt):
            if s >= 0:
                self.content[s] = t
        self.toks[self.next] = list(prompt)
        self.next += 1

    @precondition(lambda self: self.toks)
    @rule(data=st.data())
    def free(self, data):
        s = data.draw(st.sampled_from(sorted(self.toks)))
        self.pool.free_seq(s)
        del self.toks[s]

    @precondition(lambda self: self.toks)
    @rule(data=st.data())
    def fork(self, data):
        s = data.draw(st.sampled_from(sorted(self.toks)))
        self.pool.fork(s, self.next)
        self.toks[self.next] = list(self.toks[s])
        self.next += 1

    @precondition(lambda self: self.toks)
    @rule(data=st.data())
    def append(self, data):
        s = data.draw(st.sampled_from(sorted(self.toks)))
        new = data.draw(st.lists(st.integers(0, 5), min_size=1, max_size=5))
        try:
            slots, pairs = self.pool.append([(s, len(new))])
        except OutOfBlocks:
            return
        B = self.pool.block_size
        for a, b in pairs:
            for o in range(B):
                if a * B + o in self.content:
                    self.content[b * B + o] = self.content[a * B + o]
        for sl, t in zip(slots, new):
            self.content[sl] = t
        self.toks[s] += new

    @invariant()
    def consistent_and_every_sequence_reads_its_tokens(self):
        if not hasattr(self, "pool"):
            return
        self.pool.check_invariants()
        B = self.pool.block_size
        for s, toks in self.toks.items():
            blocks = self.pool.blocks(s)
            assert [self.content.get(blocks[t // B] * B + t % B) for t in range(len(toks))] == toks


PrefixCacheMachine.TestCase.settings = settings(max_examples=150, stateful_step_count=40, deadline=None)
TestPrefixCacheMachine = PrefixCacheMachine.TestCase


def test_beam_search_is_a_block_tree():
    """Slide 14: beam candidates share their common prefix like forked processes. Four beams,
    each step every beam proposes three continuations (forks), the best four survive (the rest
    are freed), and each survivor appends its token: the pool holds the tree's distinct blocks,
    far fewer than four private histories, and every beam reads its own tokens."""
    B, k = 4, 4
    p = BlockPool(200, B)
    rng = np.random.default_rng(5)
    content = {}
    p.add(0)
    slots, _ = p.append([(0, 10)])
    for s, t in zip(slots, range(10)):
        content[s] = t
    hist = {0: list(range(10))}
    beams, nxt = [0], 1
    for step in range(12):
        cands = []
        for b in beams:
            for _ in range(3):
                p.fork(b, nxt)
                hist[nxt] = list(hist[b])
                cands.append((float(rng.random()), nxt))
                nxt += 1
        for b in beams:
            p.free_seq(b)
            del hist[b]
        cands.sort(reverse=True)
        beams = [c for _, c in cands[:k]]
        for _, c in cands[k:]:
            p.free_seq(c)
            del hist[c]
        tok = {b: 100 + step * 10 + i for i, b in enumerate(beams)}
        slots, pairs = p.append([(b, 1) for b in beams])
        for a, b2 in pairs:
            for o in range(B):
                if a * B + o in content:
                    content[b2 * B + o] = content[a * B + o]
        for b, s in zip(beams, slots):
            content[s] = tok[b]
            hist[b].append(tok[b])
        p.check_invariants()
        for b in beams:
            bl = p.blocks(b)
            assert [content[bl[t // B] * B + t % B] for t in range(len(hist[b]))] == hist[b]
    used = p.num_blocks - p.num_free()
    private = sum(-(-len(hist[b]) // B) for b in beams)
    assert used < private, (used, private)
