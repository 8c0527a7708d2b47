"""Beam search as a block tree ("vLLM and PagedAttention" slide 14: beam candidates share their
common prefix the way forked processes share pages) through the native pool, copy_blocks and the
one-call decode step, against the oracle replaying the same schedule: after every step the slots and
copy-on-write pairs agree, both caches are byte-identical, and attention over the beams matches the
oracle; at the end the pool holds fewer blocks than the beams' private histories would."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.allocator import BlockPool
from paged_kv_cache_416_amd import kernels
from paged_kv_cache_416_amd.cache import PagedKVCache, to_device

from harness import TORCH_DTYPE, assert_close, cache_bytes, host_bytes, same_bytes, say

pytestmark = pytest.mark.gpu

BALANCED = -1  # PKV_PARTITION_BALANCED


@pytest.mark.parametrize("dtype,hq,hkv,P", [("f16", 8, 8, 0), ("bf16", 32, 8, 0), ("bf16", 32, 8, BALANCED)])
def test_beam_search_block_tree(dtype, hq, hkv, P):
    b = synth.beam_search(hq=hq, hkv=hkv, dtype=dtype)
    B, d, scale = b["block_size"], b["d"], b["scale"]
    dt = TORCH_DTYPE[dtype]
    c = PagedKVCache(b["num_blocks"], B, hkv, d, dt, free_order=b["free_order"])
    dev = c.device
    pool = BlockPool(b["num_blocks"], B, b["free_order"])
    kc = oracle.poisoned_cache(b["num_blocks"], hkv, B, d, dtype)
    vc = oracle.poisoned_cache(b["num_blocks"], hkv, B, d, dtype)

    # the prompt, in sequence 0
    n0 = b["prompt_k"].shape[0]
    c.add(0)
    pool.add(0)
    c.append([0], [to_device(b["prompt_k"], dt, dev)], [to_device(b["prompt_v"], dt, dev)])
    slots, _ = pool.append([(0, n0)])
    oracle.reshape_and_cache(b["prompt_k"], b["prompt_v"], kc, vc, np.array(slots, np.int64), B)
    say(f"[beam {dtype} Hq={hq} Hkv={hkv} P={P}] prompt {n0} tokens, pool {b['num_blocks']} blocks")

    beams, nxt, copies = [0], 1, []
    for t, step in enumerate(b["steps"]):
        # every live beam forks its candidates; the parents go; the highest scores survive
        cands = []
        for beam in beams:
            for _ in range(b["fanout"]):
                c.fork(beam, nxt)
                pool.fork(beam, nxt)
                cands.append(nxt)
                nxt += 1
        for beam in beams:
            c.free(beam)
            pool.free_seq(beam)
        order = np.argsort(-step["scores"], kind="stable")
        keep = step["k"].shape[0]
        beams = [cands[i] for i in order[:keep]]
        for i in order[keep:]:
            c.free(cands[i])
            pool.free_seq(cands[i])

        # one token per beam: slots and copy-on-write pairs on both sides, the copies, then the
        # decode step (the new rows written to their slots, attention over the cache holding them)
        reqs = [(s, 1) for s in beams]
        slots_n, pairs_n = c.pool.append(reqs)
        slots_o, pairs_o = pool.append(reqs)
        assert slots_n.tolist() == list(slots_o), f"step {t}: slots"
        assert [tuple(x) for x in pairs_n.tolist()] == [tuple(x) for x in pairs_o], f"step {t}: copy pairs"
        copies.append(len(pairs_o))
        if len(pairs_n):
            kernels.copy_blocks([c.k], [c.v], pairs_n)
        if pairs_o:
            oracle.copy_blocks(kc, vc, pairs_o)
        oracle.reshape_and_cache(step["k"], step["v"], kc, vc, np.array(slots_o, np.int64), B)

        tb, ctx, mx = c.tables(beams)
        q = to_device(step["q"], dt, dev)
        out = torch.full_like(q, float("nan"))
        ws = kernels.alloc_workspace(len(beams), hq, d, mx, P, dev)
        kernels.paged_attention_decode_step(out, q, to_device(step["k"], dt, dev), to_device(step["v"], dt, dev),
                                            torch.from_numpy(slots_n).to(dev), c.k, c.v, tb, ctx, mx, scale,
                                            partition_size=P, workspace=ws)
        torch.cuda.synchronize()
        same_bytes(cache_bytes(c.k), host_bytes(kc), f"step {t} K")
        same_bytes(cache_bytes(c.v), host_bytes(vc), f"step {t} V")
        tbo, ctxo = oracle.batch_tables(pool, beams)
        assert ctx.cpu().tolist() == ctxo.tolist()
        ref = oracle.paged_attention(step["q"], kc, vc, tbo, ctxo, scale, dtype)
        assert_close(out, ref, dtype, f"beam step {t}")
        pool.check_invariants()

    used = b["num_blocks"] - c.pool.num_free()
    assert used == b["num_blocks"] - pool.num_free()
    private = sum(-(-int(x) // B) for x in ctxo)
    say(f"  copies per step {copies}; blocks held {used}, private histories would hold {private}")
    # the first step copies the prompt's shared partial block for all but the last writer
    assert copies[0] == len(b["steps"][0]["k"]) - 1
    assert used < private
