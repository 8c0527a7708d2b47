"""Pins of the continuous-batching memory simulator in oracle/simulator.py.

Each check is fixed by something other than the simulator's own loop: hand-worked
timelines (written out step by step below), a closed form for the case where memory never
runs short, the pages' bounds (a 150-token answer in a 2048- or 4096-slot reservation wastes
more than 85 % of it, lesson note section 1; paged memory wastes less than one block per
sequence, lesson note section 2 and slide 11), and conservation laws of the policy."""
import numpy as np
import pytest

from oracle.simulator import FIELDS, Stalled, simulate_contiguous, simulate_paged

F = {name: i for i, name in enumerate(FIELDS)}


def rows_of(rows):
    return [tuple(r) for r in rows]


# --- hand-worked timelines -------------------------------------------------------------------

# External fragmentation (lesson note, section 1): 12 slots; r0, r1, r2 reserve 3, 6 and 3
# slots and fill the space; r0 and r2 finish after one step, leaving two 3-slot holes: 6 slots
# free, yet r3's 5-slot reservation fits nowhere until r1 ends at step 5.
FRAG = dict(arrival=[0, 0, 0, 0], prompt=[1, 1, 1, 1], output=[1, 5, 1, 1])
FRAG_CONTIG = [
    # step run wait used held free largest adm pre fin dec blocked final
    (0, 3, 1, 3, 12, 0, 0, 3, 0, 0, 0, 5, 10),
    (1, 1, 1, 2, 6, 6, 3, 0, 0, 2, 3, 5, 6),
    (2, 1, 1, 3, 6, 6, 3, 0, 0, 0, 1, 5, 6),
    (3, 1, 1, 4, 6, 6, 3, 0, 0, 0, 1, 5, 6),
    (4, 1, 1, 5, 6, 6, 3, 0, 0, 0, 1, 5, 6),
    (5, 1, 0, 1, 5, 7, 7, 1, 0, 1, 1, 0, 2),
    (6, 0, 0, 0, 0, 12, 12, 0, 0, 1, 1, 0, 0),
]
# The same requests in a pool of twelve 1-slot blocks: all four start at once.
FRAG_PAGED = [
    (0, 4, 0, 4, 4, 8, 8, 4, 0, 0, 0, 0, 12),
    (1, 1, 0, 2, 2, 10, 10, 0, 0, 3, 4, 0, 6),
    (2, 1, 0, 3, 3, 9, 9, 0, 0, 0, 1, 0, 6),
    (3, 1, 0, 4, 4, 8, 8, 0, 0, 0, 1, 0, 6),
    (4, 1, 0, 5, 5, 7, 7, 0, 0, 0, 1, 0, 6),
    (5, 0, 0, 0, 0, 12, 12, 0, 0, 1, 1, 0, 0),
]


def test_external_fragmentation_timeline():
    rows, fin = simulate_contiguous(12, 8, reserve=[3, 6, 3, 5], **FRAG)
    assert rows_of(rows) == FRAG_CONTIG
    assert fin == [1, 5, 1, 6]
    r = FRAG_CONTIG[1]  # the step that shows it: enough free slots, no hole large enough
    assert r[F["free"]] >= r[F["blocked_need"]] > r[F["largest_free"]]


def test_paged_same_requests_timeline():
    rows, fin = simulate_paged(12, 1, 0, 8, **FRAG)
    assert rows_of(rows) == FRAG_PAGED
    assert fin == [1, 5, 1, 1]


# Eviction (slide 15): four 2-slot blocks; r0 (prompt 3, output 4) and r1 (prompt 2, output 2).
# Step 1 takes the last block; at step 2 r0 needs a new block, so the newest request, r1, is
# evicted whole and waits at the head of the queue with its one generated token; it is
# admitted again (prefill of 3 tokens, 2 blocks) when r0 finishes at step 4.
EVICT = dict(arrival=[0, 0], prompt=[3, 2], output=[4, 2])
EVICT_PAGED = [
    (0, 2, 0, 5, 6, 2, 2, 2, 0, 0, 0, 0, 11),
    (1, 2, 0, 7, 8, 0, 0, 0, 0, 0, 2, 0, 11),
    (2, 1, 1, 5, 6, 2, 2, 0, 1, 0, 1, 4, 7),
    (3, 1, 1, 6, 6, 2, 2, 0, 0, 0, 1, 4, 7),
    (4, 1, 0, 3, 4, 4, 4, 1, 0, 1, 1, 0, 4),
    (5, 0, 0, 0, 0, 8, 8, 0, 0, 1, 1, 0, 0),
]
# The same requests with exact reservations (7 and 4 slots) in 8 slots: r1 waits for r0.
EVICT_CONTIG = [
    (0, 1, 1, 3, 7, 1, 1, 1, 0, 0, 0, 4, 7),
    (1, 1, 1, 4, 7, 1, 1, 0, 0, 0, 1, 4, 7),
    (2, 1, 1, 5, 7, 1, 1, 0, 0, 0, 1, 4, 7),
    (3, 1, 1, 6, 7, 1, 1, 0, 0, 0, 1, 4, 7),
    (4, 1, 0, 2, 4, 4, 4, 1, 0, 1, 1, 0, 4),
    (5, 1, 0, 3, 4, 4, 4, 0, 0, 0, 1, 0, 4),
    (6, 0, 0, 0, 0, 8, 8, 0, 0, 1, 1, 0, 0),
]


def test_eviction_timeline():
    rows, fin = simulate_paged(4, 2, 0, 8, **EVICT)
    assert rows_of(rows) == EVICT_PAGED
    assert fin == [4, 5]


def test_exact_reservation_timeline():
    rows, fin = simulate_contiguous(8, 8, reserve=[7, 4], **EVICT)
    assert rows_of(rows) == EVICT_CONTIG
    assert fin == [4, 6]


# A third request r2 (prompt 2, output 1) arrives at step 1 and waits behind the full pool. When
# r1 is evicted at step 2 it goes back ahead of r2, so r2, which would fit in the one free block,
# is not admitted: admission takes the queue head only. Both start when r0 finishes at step 4.
EVICT3 = dict(arrival=[0, 0, 1], prompt=[3, 2, 2], output=[4, 2, 1])
EVICT3_PAGED = [
    (0, 2, 0, 5, 6, 2, 2, 2, 0, 0, 0, 0, 11),
    (1, 2, 1, 7, 8, 0, 0, 0, 0, 0, 2, 2, 11),
    (2, 1, 2, 5, 6, 2, 2, 0, 1, 0, 1, 4, 7),
    (3, 1, 2, 6, 6, 2, 2, 0, 0, 0, 1, 4, 7),
    (4, 2, 0, 5, 6, 2, 2, 2, 0, 1, 1, 0, 7),
    (5, 0, 0, 0, 0, 8, 8, 0, 0, 2, 2, 0, 0),
]


def test_evicted_request_rejoins_at_the_head():
    rows, fin = simulate_paged(4, 2, 0, 8, **EVICT3)
    assert rows_of(rows) == EVICT3_PAGED
    assert fin == [4, 5, 5]


def test_watermark_exact_fit():
    """Three 2-slot blocks, one kept free: a 3-token prompt needs 2 blocks, and 2 + 1 = 3 free
    blocks admit it at once; its one decode token fits the second block's free slot."""
    rows, fin = simulate_paged(3, 2, 1, 4, [0], [3], [1])
    assert rows_of(rows) == [(0, 1, 0, 3, 4, 2, 2, 1, 0, 0, 0, 0, 4), (1, 0, 0, 0, 0, 6, 6, 0, 0, 1, 1, 0, 0)]
    assert fin == [1]


# --- closed form when memory never runs short -----------------------------------------------

def _ample(seed, n=40, B=16):
    r = np.random.default_rng(seed)
    arrival = np.sort(r.integers(0, 60, n))
    prompt = r.integers(1, 300, n)
    output = r.integers(1, 120, n)
    return arrival, prompt, output


def _closed_form(arrival, prompt, output, held_of):
    """Admitted at arrival a, decoding at a+1 .. a+O, finishing at a+O: at step t the running
    requests are those with a <= t < a+O, each holding P + (t - a) tokens."""
    T = int((arrival + output).max()) + 1
    out = []
    for t in range(T):
        run = (arrival <= t) & (t < arrival + output)
        L = prompt[run] + (t - arrival[run])
        held = int(held_of(run, L))
        out.append((t, int(run.sum()), 0, int(L.sum()), held, None, None, int((arrival == t).sum()), 0,
                    int((arrival + output == t).sum()), int(((arrival < t) & (t <= arrival + output)).sum()), 0,
                    int((prompt[run] + output[run]).sum())))
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_ample_memory_closed_form(seed):
    B = 16
    arrival, prompt, output = _ample(seed, B=B)
    N = 10 ** 5
    rows, fin = simulate_paged(N, B, 0, 10 ** 6, arrival, prompt, output)
    exp = _closed_form(arrival, prompt, output, lambda run, L: (-(-L // B) * B).sum())
    assert len(rows) == len(exp)
    for got, want in zip(rows, exp):
        for k, (a, b) in enumerate(zip(got, want)):
            if b is not None:
                assert a == b, (FIELDS[k], got, want)
        assert got[F["free"]] == N * B - got[F["held"]] == got[F["largest_free"]]
    assert fin == (arrival + output).tolist()
    reserve = prompt + output + 7
    rows, fin = simulate_contiguous(10 ** 7, 10 ** 6, arrival, prompt, output, reserve)
    exp = _closed_form(arrival, prompt, output, lambda run, L: reserve[run].sum())
    for got, want in zip(rows, exp):
        for k, (a, b) in enumerate(zip(got, want)):
            if b is not None:
                assert a == b, (FIELDS[k], got, want)
    assert fin == (arrival + output).tolist()


# --- the pages' bounds -----------------------------------------------------------------------

@pytest.mark.parametrize("R", [2048, 4096])
def test_reservation_waste_of_a_150_token_answer(R):
    """Lesson note, section 1: a request that ends after 150 tokens leaves more than 85 % of a
    2048- or 4096-token reservation unused. Its most-filled step holds P + O - 1 = 149 tokens."""
    rows, _ = simulate_contiguous(R, 1, [0], [20], [130], [R])
    best = max(r[F["used"]] / r[F["held"]] for r in rows if r[F["held"]])
    assert best == 149 / R
    assert 1 - best > 0.85
    # and the paged scheme with 16-slot blocks holds at most 15 slots it does not use
    rows, _ = simulate_paged(R // 16, 16, 0, 1, [0], [20], [130])
    assert all(0 <= r[F["held"]] - r[F["used"]] <= 15 for r in rows)


def _crowded(seed, n=120):
    r = np.random.default_rng(seed)
    arrival = np.sort(r.integers(0, 200, n))
    prompt = np.clip(np.rint(r.lognormal(np.log(200), 0.8, n)), 1, 1000).astype(int)
    output = np.clip(np.rint(r.lognormal(np.log(150), 0.8, n)), 1, 1000).astype(int)
    return arrival, prompt, output


@pytest.mark.parametrize("seed", [4, 5])
def test_paged_tail_is_under_one_block_per_sequence(seed):
    """Lesson note section 2 and slide 11: only a sequence's last block has empty slots, so the
    held but unused slots are fewer than one block per running request; with every sequence at
    400 tokens or more and 16-slot blocks that is under 4 % (15 / 400)."""
    arrival, prompt, output = _crowded(seed)
    for B in (4, 16, 32):
        rows, _ = simulate_paged(-(-8000 // B), B, 2, 64, arrival, prompt, output)
        for r in rows:
            gap = r[F["held"]] - r[F["used"]]
            assert 0 <= gap <= r[F["running"]] * (B - 1)
    rows, _ = simulate_paged(2000, 16, 0, 16, [0] * 16, [400] * 16, [50] * 16)
    assert all(r[F["held"]] - r[F["used"]] < 0.04 * r[F["held"]] for r in rows if r[F["held"]])


def test_contiguous_batch_is_capacity_over_reservation():
    """Reserving R slots per request in C slots runs at most floor(C / R) at once, and exactly
    that many while enough requests wait."""
    n, R, C = 60, 2048, 14640
    rows, _ = simulate_contiguous(C, 1000, [0] * n, [100] * n, [300] * n, [R] * n)
    assert max(r[F["running"]] for r in rows) == C // R == 7
    assert all(r[F["running"]] == 7 for r in rows if r[F["waiting"]])


# --- conservation and order ------------------------------------------------------------------

@pytest.mark.parametrize("seed", [6, 7, 8])
def test_conservation_and_order(seed):
    arrival, prompt, output = _crowded(seed)
    for kind in ("paged", "contiguous"):
        if kind == "paged":
            rows, fin = simulate_paged(300, 16, 1, 24, arrival, prompt, output)
            C = 300 * 16
        else:
            rows, fin = simulate_contiguous(4800, 24, arrival, prompt, output, np.full(len(arrival), 2048))
            C = 4800
        a = np.array(rows)
        # every generated token is decoded exactly once, even across evictions
        assert a[:, F["decoded"]].sum() == output.sum()
        assert a[:, F["finished"]].sum() == len(arrival)
        assert (a[:, F["step"]] == np.arange(len(a))).all()
        assert (a[:, F["held"]] + a[:, F["free"]] == C).all()
        assert (a[:, F["used"]] <= a[:, F["held"]]).all() and (a[:, F["used"]] <= a[:, F["final_sum"]]).all()
        assert (a[:, F["running"]] <= 24).all() and (a[:, F["largest_free"]] <= a[:, F["free"]]).all()
        # the batch changes only by admissions, evictions and finishes
        run = np.concatenate([[0], a[:, F["running"]]])
        assert (np.diff(run) == a[:, F["admitted"]] - a[:, F["preempted"]] - a[:, F["finished"]]).all()
        # a request finishes no earlier than O steps after it arrives
        assert (np.array(fin) >= arrival + output).all()
        if kind == "contiguous":
            assert a[:, F["preempted"]].sum() == 0
            # without evictions a request decodes on the O steps after its admission, and
            # admission is first come first served: admission steps follow request order
            admit = np.array(fin) - output
            assert (np.diff(admit) >= 0).all() and (admit >= arrival).all()
        else:
            assert a[:, F["preempted"]].sum() > 0  # this pool is small enough to force evictions


def test_stall_and_bad_input():
    with pytest.raises(Stalled):
        simulate_paged(20, 4, 0, 4, [0], [4], [50], max_steps=20)
    with pytest.raises(ValueError):
        simulate_paged(2, 4, 0, 4, [0], [4], [5])  # 9 tokens never fit in 2 blocks of 4
    with pytest.raises(ValueError):
        simulate_contiguous(100, 4, [0], [4], [5], [8])  # reservation below P + O
    with pytest.raises(ValueError):
        simulate_paged(10, 4, 0, 4, [3, 1], [1, 1], [1, 1])  # arrivals out of order
