"""The native memory simulator (pkv_sim_paged / pkv_sim_contiguous, over the library's own block
pool) against the oracle's (oracle/simulator.py, over the Python allocator model): every trace
row and every finish step equal, on seeded request mixes sized so that the pool runs short
(evictions) and the contiguous range fragments. Host only: no GPU is used."""
import numpy as np
import pytest

import synth
from oracle import simulator as ref
from paged_kv_cache_416_amd import sim
from paged_kv_cache_416_amd._lib import PKV_EINVAL, PkvError


def _same(native, oracle):
    t, f = native
    rows, fin = oracle
    assert t.shape == (len(rows), len(ref.FIELDS))
    bad = np.argwhere(t != np.array(rows, dtype=np.int64))
    assert not len(bad), f"first difference at step {bad[0][0]}, field {ref.FIELDS[bad[0][1]]}"
    assert f.tolist() == fin


CASES = [
    # seed, n, prompt median, output median, max context, rate, blocks, block size, watermark, batch
    (11, 150, 60, 80, 512, 0.5, 160, 16, 2, 32),
    (12, 150, 60, 80, 512, None, 96, 16, 0, 64),
    (13, 120, 30, 40, 256, 1.0, 300, 4, 3, 24),
    (14, 100, 100, 100, 1024, 0.2, 140, 32, 1, 16),
    (15, 200, 10, 20, 128, 2.0, 64, 8, 0, 8),
]


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_paged_matches_oracle(case):
    seed, n, pm, om, ctx, rate, N, B, W, mb = case
    a, p, o = synth.serving_requests(seed, n, pm, om, 1.0, ctx, rate)
    nat = sim.simulate_paged(N, B, W, mb, a, p, o)
    _same(nat, ref.simulate_paged(N, B, W, mb, a, p, o))
    if seed != 13:
        assert nat[0][:, ref.FIELDS.index("preempted")].sum() > 0  # the pool ran short


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_contiguous_matches_oracle(case):
    seed, n, pm, om, ctx, rate, N, B, W, mb = case
    a, p, o = synth.serving_requests(seed, n, pm, om, 1.0, ctx, rate)
    r = np.random.default_rng(seed)
    for reserve in (np.full(n, ctx), p + o + r.integers(0, 64, n)):  # the maximum length, or near-exact
        nat = sim.simulate_contiguous(N * B, mb, a, p, o, reserve)
        _same(nat, ref.simulate_contiguous(N * B, mb, a, p, o, reserve))
    blocked = nat[0][:, ref.FIELDS.index("blocked_need")]
    free = nat[0][:, ref.FIELDS.index("free")]
    largest = nat[0][:, ref.FIELDS.index("largest_free")]
    if seed in (11, 12):  # these mixes show external fragmentation with near-exact reservations
        assert ((blocked > 0) & (free >= blocked) & (largest < blocked)).any()


def test_hand_cases():
    from tests.test_oracle_sim import EVICT, EVICT3, EVICT3_PAGED, EVICT_CONTIG, EVICT_PAGED, FRAG, FRAG_CONTIG, FRAG_PAGED
    t, f = sim.simulate_paged(12, 1, 0, 8, **FRAG)
    assert [tuple(r) for r in t.tolist()] == FRAG_PAGED
    t, f = sim.simulate_contiguous(12, 8, reserve=[3, 6, 3, 5], **FRAG)
    assert [tuple(r) for r in t.tolist()] == FRAG_CONTIG
    t, f = sim.simulate_paged(4, 2, 0, 8, **EVICT)
    assert [tuple(r) for r in t.tolist()] == EVICT_PAGED
    t, f = sim.simulate_contiguous(8, 8, reserve=[7, 4], **EVICT)
    assert [tuple(r) for r in t.tolist()] == EVICT_CONTIG
    t, f = sim.simulate_paged(4, 2, 0, 8, **EVICT3)
    assert [tuple(r) for r in t.tolist()] == EVICT3_PAGED


def test_empty_and_single():
    t, f = sim.simulate_paged(4, 16, 0, 4, [], [], [])
    assert t.tolist() == [[0, 0, 0, 0, 0, 64, 64, 0, 0, 0, 0, 0, 0]] and f.tolist() == []
    assert t.tolist() == [list(r) for r in ref.simulate_paged(4, 16, 0, 4, [], [], [])[0]]
    t, f = sim.simulate_contiguous(100, 4, [5], [3], [2], [5])
    _same((t, f), ref.simulate_contiguous(100, 4, [5], [3], [2], [5]))
    assert f.tolist() == [7] and len(t) == 8


@pytest.mark.parametrize("call", [
    lambda: sim.simulate_paged(2, 4, 0, 4, [0], [4], [5]),  # 9 tokens never fit 2 blocks of 4
    lambda: sim.simulate_paged(10, 4, 10, 4, [0], [1], [1]),  # watermark leaves no room
    lambda: sim.simulate_paged(10, 4, 0, 4, [3, 1], [1, 1], [1, 1]),  # arrivals out of order
    lambda: sim.simulate_paged(10, 4, 0, 4, [0], [0], [1]),  # empty prompt
    lambda: sim.simulate_paged(10, 4, 0, 0, [0], [1], [1]),  # no batch
    lambda: sim.simulate_paged(20, 4, 0, 4, [0], [4], [50], max_steps=20),  # does not drain
    lambda: sim.simulate_contiguous(100, 4, [0], [4], [5], [8]),  # reservation below P + O
    lambda: sim.simulate_contiguous(100, 4, [0], [4], [5], [101]),  # reservation above capacity
])
def test_errors(call):
    with pytest.raises(PkvError) as e:
        call()
    assert e.value.code == PKV_EINVAL


def test_summary_figures():
    """The summary's shares come straight from the trace columns."""
    a, p, o = synth.serving_requests(16, 300, 100, 120, 1.0, 1024, None)
    t, _ = sim.simulate_paged(400, 16, 4, 256, a, p, o)
    s = sim.summarize(t, 400 * 16)
    col = {n: t[:, k] for k, n in enumerate(sim.FIELDS)}
    assert s["useful_of_held"] == col["used"].sum() / col["held"].sum()
    assert s["decoded"] == o.sum() and s["steps"] == len(t)
    tc, _ = sim.simulate_contiguous(400 * 16, 256, a, p, o, np.full(300, 1024))
    sc = sim.summarize(tc, 400 * 16)
    # reserving the maximum length holds far more than it uses; the paged pool wastes under a block each
    assert sc["useful_of_held_saturated"] < 0.5 < 0.9 < s["useful_of_held_saturated"]
    assert s["mean_batch_saturated"] > 2 * sc["mean_batch_saturated"]
