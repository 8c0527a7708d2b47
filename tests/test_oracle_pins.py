"""Pins of the CPU oracle against things other than itself.

Each pin goes through a route the oracle does not use: a library routine
(torch's scaled_dot_product_attention in float64, numpy's / torch's own
float16 and bfloat16 decoders), a closed form, a worked example printed on
the pages, or an invariant of the mathematics. Placement of tokens into
blocks in these tests is done with numpy reshapes and fancy indexing, not
with the oracle's index formulas.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa(q, k, v, scale):
    """Library reference: q [S,Hq,D], k/v [S,Hq,T,D] float64 -> [S,Hq,D]."""
    qt = torch.from_numpy(q)[:, :, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qt, torch.from_numpy(k), torch.from_numpy(v),
                                                           scale=scale)
    return out[:, :, 0, :].numpy()


def _place(streams_k, streams_v, tables, num_blocks, hkv, B, d, dtype):
    """Put each sequence's token rows into the blocks its table names (numpy reshapes only)."""
    kc = oracle.poisoned_cache(num_blocks, hkv, B, d, dtype)
    vc = oracle.poisoned_cache(num_blocks, hkv, B, d, dtype)
    for s, (ks, vs) in enumerate(zip(streams_k, streams_v)):
        n = ks.shape[0]
        nb = -(-n // B)
        pad = nb * B - n
        for src, dst in ((ks, kc), (vs, vc)):
            full = np.concatenate([src, np.zeros((pad, hkv, d), src.dtype)]) if pad else src
            tiles = full.reshape(nb, B, hkv, d).transpose(0, 2, 1, 3)  # [nb, Hkv, B, D]
            for j in range(nb):
                keep = B if j < nb - 1 or pad == 0 else B - pad
                dst[tables[s][j], :, :keep, :] = tiles[j, :, :keep, :]
    return kc, vc


def _random_case(rng, S, hq, hkv, d, B, max_ctx, dtype, vscale=1.0):
    ctx = rng.integers(1, max_ctx + 1, size=S).astype(np.int32)
    nbs = [-(-int(c) // B) for c in ctx]
    N = sum(nbs) + 3
    perm = rng.permutation(N).astype(np.int32)
    maxb = max(nbs)
    tables = np.full((S, maxb), -1, np.int32)
    pos = 0
    for s in range(S):
        tables[s, :nbs[s]] = perm[pos:pos + nbs[s]]
        pos += nbs[s]
    ks = [synth.normal(rng, (int(c), hkv, d), vscale, dtype) for c in ctx]
    vs = [synth.normal(rng, (int(c), hkv, d), vscale, dtype) for c in ctx]
    q = synth.normal(rng, (S, hq, d), vscale, dtype)
    kc, vc = _place(ks, vs, tables, N, hkv, B, d, dtype)
    return q, ks, vs, kc, vc, tables, ctx


def _expected(q, ks, vs, ctx, hq, scale, dtype):
    """Library SDPA per sequence over its logical stream, GQA heads repeated (head h reads h // G)."""
    S = q.shape[0]
    out = np.zeros(q.shape, np.float64)
    for s in range(S):
        k = synth.storage_to_f64(ks[s], dtype)  # [T, Hkv, D]
        v = synth.storage_to_f64(vs[s], dtype)
        G = hq // k.shape[1]
        k = np.repeat(k.transpose(1, 0, 2), G, axis=0)[None]  # [1, Hq, T, D]
        v = np.repeat(v.transpose(1, 0, 2), G, axis=0)[None]
        out[s] = _sdpa(synth.storage_to_f64(q[s:s + 1], dtype), k, v, scale)[0]
    return out


# ---------------------------------------------------------------- element decoders

def test_f16_decoder_matches_numpy_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits.view(np.float16), "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decoder_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_rounding_of_inputs_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    mine = synth.to_storage(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


# ---------------------------------------------------------------- attention vs library

@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), S=st.integers(1, 4), hkv=st.integers(1, 3), G=st.sampled_from([1, 2, 4]),
       d=st.sampled_from([8, 16, 64]), B=st.sampled_from([1, 4, 8, 16]), max_ctx=st.integers(1, 64),
       dtype=st.sampled_from(["f32", "f16", "bf16"]))
def test_paged_attention_equals_library_sdpa(seed, S, hkv, G, d, B, max_ctx, dtype):
    rng = np.random.default_rng(seed)
    hq = hkv * G
    q, ks, vs, kc, vc, tables, ctx = _random_case(rng, S, hq, hkv, d, B, max_ctx, dtype)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    got = oracle.paged_attention(q, kc, vc, tables, ctx, scale, dtype)
    ref = _expected(q, ks, vs, ctx, hq, scale, dtype)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), S=st.integers(1, 3), G=st.sampled_from([1, 2]),
       B=st.sampled_from([2, 8, 16]), P_blocks=st.integers(1, 4), max_ctx=st.integers(1, 150),
       dtype=st.sampled_from(["f32", "bf16"]))
def test_split_merge_equals_unsplit(seed, S, G, B, P_blocks, max_ctx, dtype):
    """The partition + log-sum-exp merge is an identity: split and unsplit agree to rounding."""
    rng = np.random.default_rng(seed)
    q, ks, vs, kc, vc, tables, ctx = _random_case(rng, S, 2 * G, 2, 16, B, max_ctx, dtype, vscale=2.0)
    a = oracle.paged_attention(q, kc, vc, tables, ctx, 0.25, dtype)
    b = oracle.paged_attention(q, kc, vc, tables, ctx, 0.25, dtype, partition_size=P_blocks * B)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-14)


def test_contiguous_attention_equals_library_sdpa():
    rng = np.random.default_rng(7)
    S, hq, hkv, d, lmax = 3, 4, 2, 32, 40
    ctx = np.array([1, 17, 40], np.int32)
    k = synth.normal(rng, (S, hkv, lmax, d), 1.0, "f16")
    v = synth.normal(rng, (S, hkv, lmax, d), 1.0, "f16")
    q = synth.normal(rng, (S, hq, d), 1.0, "f16")
    got = oracle.contiguous_attention(q, k, v, ctx, 0.2, "f16")
    ks = [k[s, :, :ctx[s]].transpose(1, 0, 2) for s in range(S)]
    vs = [v[s, :, :ctx[s]].transpose(1, 0, 2) for s in range(S)]
    ref = _expected(q, ks, vs, ctx, hq, 0.2, "f16")
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- closed forms / special cases

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_token_returns_its_value_exactly(dtype):
    rng = np.random.default_rng(1)
    q, ks, vs, kc, vc, tables, _ = _random_case(rng, 3, 4, 2, 64, 16, 40, dtype)
    ctx = np.ones(3, np.int32)
    got = oracle.paged_attention(q, kc, vc, tables, ctx, 0.125, dtype)
    for s in range(3):
        v0 = synth.storage_to_f64(vs[s][0], dtype)  # [Hkv, D]
        assert np.array_equal(got[s], np.repeat(v0, 2, axis=0))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    q, ks, vs, kc, vc, tables, ctx = _random_case(rng, 3, 2, 2, 16, 8, 50, "f32")
    q[:] = 0
    got = oracle.paged_attention(q, kc, vc, tables, ctx, 0.5, "f32")
    for s in range(3):
        np.testing.assert_allclose(got[s], vs[s].astype(np.float64).mean(axis=0), rtol=1e-13, atol=1e-15)


def test_two_tokens_sigmoid_weights():
    """With two keys the weights are sigmoid(a - b) and sigmoid(b - a)."""
    d, B = 4, 2
    q = np.array([[[1.0, 2.0, -1.0, 0.5]]], np.float32)
    k = np.array([[[0.5, 0.25, 1.0, -2.0]], [[-1.0, 1.0, 0.0, 4.0]]], np.float32)  # [2, 1, 4]
    v = np.array([[[1.0, 0.0, 3.0, -1.0]], [[0.0, 2.0, -3.0, 5.0]]], np.float32)
    kc, vc = _place([k], [v], [[0]], 1, 1, B, d, "f32")
    scale = 0.75
    a = scale * float(q[0, 0] @ k[0, 0])
    b = scale * float(q[0, 0] @ k[1, 0])
    wa = 1.0 / (1.0 + math.exp(b - a))
    ref = wa * v[0, 0].astype(np.float64) + (1 - wa) * v[1, 0].astype(np.float64)
    got = oracle.paged_attention(q, kc, vc, np.array([[0]], np.int32), np.array([2], np.int32), scale, "f32")
    np.testing.assert_allclose(got[0, 0], ref, rtol=1e-14, atol=1e-15)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    T, d, B = 37, 16, 8
    k = np.repeat(synth.normal(rng, (1, 1, d), 1.0, "f32"), T, axis=0)
    v = synth.normal(rng, (T, 1, d), 1.0, "f32")
    tbl = [list(rng.permutation(6)[:5])]
    kc, vc = _place([k], [v], tbl, 6, 1, B, d, "f32")
    q = synth.normal(rng, (1, 1, d), 3.0, "f32")
    got = oracle.paged_attention(q, kc, vc, np.array(tbl, np.int32), np.array([T], np.int32), 1.0, "f32")
    np.testing.assert_allclose(got[0, 0], v[:, 0].astype(np.float64).mean(0), rtol=1e-12, atol=1e-14)


def test_empty_context_gives_zeros():
    q = np.ones((2, 2, 8), np.float32)
    kc = oracle.poisoned_cache(2, 2, 4, 8, "f32")
    got = oracle.paged_attention(q, kc, kc.copy(), np.array([[0], [1]], np.int32), np.array([0, 0], np.int32),
                                 1.0, "f32")
    assert np.array_equal(got, np.zeros_like(got))


def test_unused_slots_and_padding_are_never_read():
    """NaN in every unwritten slot and -1 / INT32_MAX in table padding leave results finite."""
    rng = np.random.default_rng(4)
    q, ks, vs, kc, vc, tables, ctx = _random_case(rng, 4, 2, 2, 16, 16, 70, "f16")
    for pad in (-1, 2**31 - 1):
        t2 = np.concatenate([tables, np.full((4, 3), pad, np.int32)], axis=1)
        t2[t2 == -1] = pad
        got = oracle.paged_attention(q, kc, vc, t2, ctx, 0.25, "f16")
        assert np.isfinite(got).all()
        np.testing.assert_allclose(got, _expected(q, ks, vs, ctx, 2, 0.25, "f16"), rtol=1e-12, atol=1e-13)


def test_physical_permutation_invariance():
    """Relabelling physical blocks (moving the bytes, rewriting the tables) changes nothing."""
    rng = np.random.default_rng(5)
    q, ks, vs, kc, vc, tables, ctx = _random_case(rng, 3, 4, 2, 16, 8, 60, "bf16")
    N = kc.shape[0]
    perm = rng.permutation(N)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    a = oracle.paged_attention(q, kc, vc, tables, ctx, 0.3, "bf16")
    b = oracle.paged_attention(q, kc2, vc2, t2, ctx, 0.3, "bf16")
    assert np.array_equal(a, b)


def test_gqa_grouping_matches_repeated_heads():
    """Query head h reads KV head h // G: same as MHA over KV heads repeated G times in a row."""
    rng = np.random.default_rng(6)
    G, hkv, d, B = 4, 2, 16, 8
    q, ks, vs, kc, vc, tables, ctx = _random_case(rng, 2, G * hkv, hkv, d, B, 30, "f32")
    got = oracle.paged_attention(q, kc, vc, tables, ctx, 0.5, "f32")
    kr, vr = np.repeat(kc, G, axis=1), np.repeat(vc, G, axis=1)
    mha = oracle.paged_attention(q, kr, vr, tables, ctx, 0.5, "f32")
    assert np.array_equal(got, mha)


def test_invalid_table_entry_rejected():
    q = np.ones((1, 1, 4), np.float32)
    kc = np.zeros((2, 1, 4, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.paged_attention(q, kc, kc, np.array([[5]], np.int32), np.array([3], np.int32), 1.0, "f32")


# ---------------------------------------------------------------- pages' worked examples

def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_lesson_note_block_table_example():
    g = _load("lesson_note_block_table.json")
    B = g["block_size"]
    phys = g["physical_blocks"]
    # free order that hands out 7, 2, 11 first, the rest afterwards
    rest = [b for b in range(16) if b not in phys]
    pool = oracle.BlockPool(16, B, phys + rest)
    pool.add(0)
    slots, pairs = pool.append([(0, g["num_tokens"])])
    assert pairs == []
    assert pool.blocks(0) == phys
    for b, rc in g["ref_counts"].items():
        assert pool.ref[int(b)] == rc
    for t, sl in g["derived_under_slot_rule"]["slots"].items():
        assert slots[int(t)] == sl
    for j, (a, z) in enumerate(g["logical_blocks"]):
        assert {slots[t] // B for t in range(a, z + 1)} == {phys[j]}
    assert g["num_tokens"] - (len(phys) - 1) * B == g["derived_under_slot_rule"]["tokens_in_last_block"]


def test_slides_table_with_unallocated_entry():
    """Slide 10: logical blocks 0-2 sit in physical blocks 7, 1 and 3, and logical block 3 has no
    physical block yet; the 4th entry is never read."""
    g = _load("slides_block_table.json")
    B = g["block_size"]
    alloc = [b for b in g["physical_blocks"] if b is not None]
    rng = np.random.default_rng(8)
    n = 3 * B - 5
    k = synth.normal(rng, (n, 1, 8), 1.0, "f32")
    v = synth.normal(rng, (n, 1, 8), 1.0, "f32")
    kc, vc = _place([k], [v], [alloc], 8, 1, B, 8, "f32")
    q = synth.normal(rng, (1, 1, 8), 1.0, "f32")
    ref = _expected(q, [k], [v], [n], 1, 0.4, "f32")
    for pad in (-1, 2**31 - 1, 10**6):
        tbl = np.array([alloc + [pad]], np.int32)
        got = oracle.paged_attention(q, kc, vc, tbl, np.array([n], np.int32), 0.4, "f32")
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_blog_block_table_example():
    g = _load("blog_block_table.json")
    B, phys = g["block_size"], g["physical_blocks"]
    N = max(phys) + 1
    rest = [b for b in range(N) if b not in phys]
    pool = oracle.BlockPool(N, B, phys + rest)
    pool.add(0)
    slots, _ = pool.append([(0, 48)])
    for j, (a, z) in enumerate(g["logical_tokens"]):
        assert [slots[t] for t in range(a, z + 1)] == list(range(phys[j] * B, phys[j] * B + B))
    # every block is full, so the next token needs a new block
    assert len(pool.blocks(0)) == 3 and pool.length(0) == 48
    pool.append([(0, 1)])
    assert len(pool.blocks(0)) == 4


def test_slide11_new_block_only_when_last_fills():
    """From a state with one free slot in the last block, step 1 allocates nothing and step 2 one block."""
    B = 16
    pool = oracle.BlockPool(8, B)
    pool.add(0)
    pool.append([(0, 2 * B - 1)])  # prefill leaves one free slot
    free0 = pool.num_free()
    s1, _ = pool.append([(0, 1)])
    assert pool.num_free() == free0
    s2, _ = pool.append([(0, 1)])
    assert pool.num_free() == free0 - 1
    assert s1[0] // B == pool.blocks(0)[1] and s2[0] // B == pool.blocks(0)[2] and s2[0] % B == 0


def test_slides_800kb_per_token():
    g = _load("slides_kv_bytes.json")
    heads, d = 40, 128
    assert heads * d == g["hidden"]
    per_layer = synth.kv_bytes_per_token(heads, d, g["bytes_per_element"])
    assert per_layer == 20480
    assert per_layer * g["num_layers"] == g["bytes_per_token_all_layers"]
    per_token = per_layer * g["num_layers"]
    assert per_token == 800 * g["kilobyte"]
    assert per_token * g["request_tokens"] == g["request_gigabytes"] * 1000 * 2**20


# ---------------------------------------------------------------- cache writes and copies

def test_reshape_and_cache_logical_gather_and_poison():
    rng = np.random.default_rng(9)
    B, hkv, d, N = 8, 3, 16, 12
    pool = oracle.BlockPool(N, B, rng.permutation(N))
    kc = oracle.poisoned_cache(N, hkv, B, d, "f16")
    vc = oracle.poisoned_cache(N, hkv, B, d, "f16")
    lens = [5, 19, 8]
    streams = {}
    for s, n in enumerate(lens):
        pool.add(s)
        k = synth.normal(rng, (n, hkv, d), 1.0, "f16")
        v = synth.normal(rng, (n, hkv, d), 1.0, "f16")
        slots, _ = pool.append([(s, n)])
        oracle.reshape_and_cache(k, v, kc, vc, np.array(slots), B)
        streams[s] = (k, v)
    written = np.zeros(N * B, bool)
    for s, n in enumerate(lens):
        blocks = pool.blocks(s)
        # gather with numpy fancy indexing: token t lives in block blocks[t // B], row t % B
        t = np.arange(n)
        bk = np.array(blocks)[t // B]
        gk = kc[bk, :, t % B, :]
        gv = vc[bk, :, t % B, :]
        assert np.array_equal(gk.view(np.uint16), streams[s][0].view(np.uint16))
        assert np.array_equal(gv.view(np.uint16), streams[s][1].view(np.uint16))
        written[bk * B + t % B] = True
    flat = kc.transpose(0, 2, 1, 3).reshape(N * B, -1).view(np.uint16)
    assert (flat[~written] == 0x7E00).all()


def test_reshape_and_cache_skips_negative_slots():
    kc = oracle.poisoned_cache(2, 1, 4, 4, "f32")
    vc = kc.copy()
    before = kc.copy()
    k = np.ones((3, 1, 4), np.float32)
    oracle.reshape_and_cache(k, k, kc, vc, np.array([-1, 5, -7]), 4)
    changed = ~np.isnan(kc)
    assert changed.sum() == 4 and (kc[1, 0, 1] == 1).all()
    assert np.isnan(before).all()
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(k, k, kc, vc, np.array([0, 8, 1]), 4)


def test_copy_blocks_whole_block_bytes():
    rng = np.random.default_rng(10)
    kc = synth.normal(rng, (6, 2, 4, 8), 1.0, "bf16")
    vc = synth.normal(rng, (6, 2, 4, 8), 1.0, "bf16")
    k0, v0 = kc.copy(), vc.copy()
    oracle.copy_blocks(kc, vc, [(1, 4), (3, 0)])
    assert np.array_equal(kc[4], k0[1]) and np.array_equal(vc[4], v0[1])
    assert np.array_equal(kc[0], k0[3]) and np.array_equal(vc[0], v0[3])
    for b in (1, 2, 3, 5):
        assert np.array_equal(kc[b], k0[b]) and np.array_equal(vc[b], v0[b])


# ---------------------------------------------------------------- prefill (chunked, causal)

@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), S=st.integers(1, 3), hkv=st.integers(1, 2), G=st.sampled_from([1, 2, 4]),
       d=st.sampled_from([8, 16]), B=st.sampled_from([1, 4, 16]), max_ctx=st.integers(1, 48),
       dtype=st.sampled_from(["f32", "bf16"]))
def test_paged_prefill_equals_library_causal_sdpa(seed, S, hkv, G, d, B, max_ctx, dtype):
    """Each sequence's last n_s tokens as queries, causal over its whole context (earlier tokens
    included): the oracle equals torch's scaled_dot_product_attention in float64 with an explicit
    boolean mask (query at position p sees keys 0..p), the cases placed into blocks by numpy."""
    rng = np.random.default_rng(seed)
    hq = hkv * G
    _, ks, vs, kc, vc, tables, ctx = _random_case(rng, S, hq, hkv, d, B, max_ctx, dtype)
    n = np.array([int(rng.integers(0, c + 1)) for c in ctx], np.int32)
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = synth.normal(rng, (int(qs[-1]), hq, d), 1.0, dtype)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    got = oracle.paged_prefill(q, kc, vc, tables, ctx, qs, scale, dtype)
    for s in range(S):
        if n[s] == 0:
            continue
        k = np.repeat(synth.storage_to_f64(ks[s], dtype).transpose(1, 0, 2), G, axis=0)[None]  # [1, Hq, T, D]
        v = np.repeat(synth.storage_to_f64(vs[s], dtype).transpose(1, 0, 2), G, axis=0)[None]
        qq = synth.storage_to_f64(q[qs[s]:qs[s + 1]], dtype).transpose(1, 0, 2)[None]  # [1, Hq, n, D]
        pos = ctx[s] - n[s] + np.arange(n[s])
        mask = torch.from_numpy(pos[:, None] >= np.arange(ctx[s])[None, :])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qq), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=scale)
        np.testing.assert_allclose(got[qs[s]:qs[s + 1]], ref[0].numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-13)


def test_prefill_of_one_query_is_decode_and_whole_prompt_is_causal():
    """n_s = 1 is decode attention; a fresh prompt (n_s = ctx) has its first query return its
    own value row exactly (one key)."""
    rng = np.random.default_rng(3)
    q1, ks, vs, kc, vc, tables, ctx = _random_case(rng, 3, 4, 2, 16, 4, 30, "f32")
    one = oracle.paged_prefill(q1, kc, vc, tables, ctx, np.arange(4, dtype=np.int32), 0.25, "f32")
    np.testing.assert_array_equal(one, oracle.paged_attention(q1, kc, vc, tables, ctx, 0.25, "f32"))
    qs = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    qa = synth.normal(rng, (int(qs[-1]), 4, 16), 1.0, "f32")
    full = oracle.paged_prefill(qa, kc, vc, tables, ctx, qs, 0.25, "f32")
    for s in range(3):
        first = synth.storage_to_f64(vs[s][0], "f32")  # [Hkv, D]
        np.testing.assert_array_equal(full[qs[s]], np.repeat(first, 2, axis=0))
