"""The oracle replays every workload recipe (reduced sizes) and the results obey the recipes' invariants."""
import numpy as np
import pytest

import oracle
import synth


def _gather_dense(st, w):
    """Each batch sequence's keys/values gathered through its table with numpy fancy indexing."""
    B = w.block_size
    out = []
    for s in w.batch:
        blocks = np.array(st.pool.blocks(s))
        n = st.pool.length(s)
        t = np.arange(n)
        out.append((st.k_cache[blocks[t // B], :, t % B, :], st.v_cache[blocks[t // B], :, t % B, :]))
    return out


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


@pytest.mark.parametrize("make", [
    lambda: synth.tiny(),
    lambda: synth.llama13b(num_seqs=3, ctx_range=(20, 90)),
    lambda: synth.block_sweep(block_size=8, num_seqs=3, ctx_range=(10, 60)),
    lambda: synth.gqa_shared_prefix(num_seqs=5, prefix=48, median=20, cap=80, partition_size=32),
    lambda: synth.gqa_shared_prefix(num_seqs=3, prefix=40, median=20, cap=60, partition_size=32),
    lambda: synth.parallel_sampling(prompts=2, n=4, prompt_len=32, max_private=20, hkv=2, d=64),
])
def test_replay_reproduces_token_streams(make):
    w = make()
    st = oracle.replay(w)
    st.pool.check_invariants()
    streams = w.token_streams()
    ctx = w.final_lengths()
    for i, ((gk, gv), (k, v)) in enumerate(zip(_gather_dense(st, w), streams)):
        assert gk.shape[0] == ctx[i]
        assert np.array_equal(_bits(gk), _bits(k)) and np.array_equal(_bits(gv), _bits(v))
    out = oracle.attention_of(st, w)
    assert np.isfinite(out).all()


def test_shared_prefix_is_one_set_of_blocks():
    w = synth.gqa_shared_prefix(num_seqs=6, prefix=64, median=10, cap=40)
    st = oracle.replay(w)
    pre = [st.pool.blocks(s)[:4] for s in w.batch]
    assert all(p == pre[0] for p in pre)
    assert all(st.pool.ref[b] == 6 for b in pre[0])


def test_parallel_sampling_copies_once_per_writing_branch_but_last():
    w = synth.parallel_sampling(prompts=3, n=4, prompt_len=32, max_extra=15, max_private=5, hkv=2, d=64)
    st = oracle.replay(w)
    priv = np.array(w.notes["private"])
    first = st.step_pairs[len(st.step_pairs) - w.notes["steps"]] if w.notes["steps"] else []
    # step 1: in each prompt, k writing branches make min(k, n-1) copies of the shared partial block
    writers = (priv > 0).sum(axis=1)
    assert len(first) == int(np.minimum(writers, 3).sum())
    # afterwards no step copies anything: copy-on-write duplicates a shared last block, once
    for pairs in st.step_pairs[len(st.step_pairs) - w.notes["steps"] + 1:]:
        assert pairs == []


def test_split_partitions_agree_with_unsplit_on_recipe():
    w = synth.gqa_shared_prefix(num_seqs=4, prefix=32, median=40, cap=100, partition_size=16)
    st = oracle.replay(w)
    a = oracle.attention_of(st, w, 0)
    b = oracle.attention_of(st, w, 16)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-14)


def test_recipes_are_deterministic():
    a, b = synth.llama13b(num_seqs=2, ctx_range=(5, 30)), synth.llama13b(num_seqs=2, ctx_range=(5, 30))
    assert np.array_equal(a.free_order, b.free_order) and np.array_equal(a.q, b.q)
    for (ka, va), (kb, vb) in zip(a.token_streams(), b.token_streams()):
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)


def test_full_size_recipe_shapes():
    """Sizes of the full recipes, from their lengths alone (no value draws needed)."""
    import math
    r = np.random.default_rng([2, 1])
    lens = r.integers(128, 2049, size=30)
    blocks = sum(-(-int(c) // 16) for c in lens)
    assert 30 * 128 / 16 <= blocks <= 30 * 128
    assert math.ceil(1.1 * blocks) > blocks


def test_prefix_cache_requests_read_their_own_rows():
    """Prefix-cache workload: cached prompt tokens are never written, yet every live request's
    attention through the oracle's cache equals dense attention over that request's own prompt
    and decode rows (float64, 1e-12), and later requests did find their system prompt's blocks."""
    w = synth.prefix_cache_requests()
    st = oracle.replay(w)
    assert sum(st.cached_tokens) > 0 and st.cached_tokens[0] == 0
    ref = oracle.attention_of(st, w)
    rows = {op[1]: (op[3], op[4]) for op in w.ops if op[0] == "prompt"}
    last = {sid: (k, v) for sid, k, v in w.ops[-1][1]}
    q = synth.storage_to_f64(w.q, w.dtype)
    G = w.num_q_heads // w.num_kv_heads
    for i, sid in enumerate(w.batch):
        k = synth.storage_to_f64(np.concatenate([rows[sid][0], last[sid][0]]), w.dtype)
        v = synth.storage_to_f64(np.concatenate([rows[sid][1], last[sid][1]]), w.dtype)
        for h in range(w.num_q_heads):
            x = np.float64(w.scale) * (k[:, h // G, :] @ q[i, h])
            p = np.exp(x - x.max())
            dense = (p[:, None] * v[:, h // G, :]).sum(0) / p.sum()
            assert np.allclose(ref[i, h], dense, rtol=1e-12, atol=1e-14)
