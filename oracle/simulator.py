"""Continuous-batching memory simulator -- TEST INFRASTRUCTURE ONLY (pure Python).

Simulates only the memory side of iteration-level scheduling ("Week 22 Day 2" lesson note,
section 4: at every decode step finished sequences leave and free their memory at once, and
waiting requests are admitted and prefilled into the running batch) under two schemes that
hold the same number of token slots:

  * paged: the block pool of ``oracle.allocator`` (slides 10-12: fixed-size blocks from one
    pool, a block allocated only once the last one has no free slot); when a decode step
    cannot get its blocks, the newest running request is evicted whole and waits again at the
    head of the queue (slide 15: requests are served in arrival order, and under memory
    pressure the latest arrival leaves entirely; it comes back by recomputation);
  * contiguous: each admitted request reserves one contiguous run of ``reserve`` slots, placed
    first-fit in a linear address space and released on finish (the lesson note, section 1:
    reservation for the maximum length, and holes left by requests that finish at different
    times; slide 6: reservation, internal and external fragmentation).

Readings (the pages give the policy in words only):
  * a step runs, in order: arrivals join the queue tail; every running request decodes one
    token (its key/value state is appended); requests that reached their output length finish
    and are freed; the queue head is admitted while it fits and the batch is below
    ``max_batch``, its prompt (plus any tokens generated before an eviction) written by the
    prefill; the state is then recorded;
  * a request with prompt P and output O holds P tokens after its prefill and P + O after its
    O-th decode step, at which it finishes; a fresh request admitted at step t finishes at
    step t + O if it is never evicted;
  * admission is strictly in queue order (no request overtakes a head that does not fit); paged
    admission also leaves ``watermark`` blocks free;
  * an evicted request keeps the tokens it generated and recomputes them in its next prefill.

Each recorded step is one row of the integers named in FIELDS:
  running, waiting    requests in the batch and in the queue after admission
  used                key/value slots holding a real token (sum of running lengths)
  held                slots the scheme has given to running requests
  free, largest_free  slots not held, and the largest run of them one request could take
  admitted, preempted, finished, decoded
                      requests admitted, evicted, finished and decoding in this step
  blocked_need        slots the queue head asked for when admission stopped for memory, else 0
  final_sum           sum of the final lengths (P + O) of the running requests
"""
from __future__ import annotations

from collections import deque

from .allocator import BlockPool, OutOfBlocks

FIELDS = ("step", "running", "waiting", "used", "held", "free", "largest_free", "admitted", "preempted",
          "finished", "decoded", "blocked_need", "final_sum")


class Stalled(Exception):
    """The requests did not all finish within max_steps."""


class _PagedMemory:
    def __init__(self, num_blocks, block_size, watermark):
        self.pool = BlockPool(num_blocks, block_size)
        self.B = block_size
        self.N = num_blocks
        self.watermark = watermark

    def need(self, r, tokens):
        return -(-tokens // self.B) * self.B

    def admit(self, r, tokens):
        if self.pool.num_free() < -(-tokens // self.B) + self.watermark:
            return False
        self.pool.add(r)
        self.pool.append([(r, tokens)])
        return True

    def grow(self, running):
        self.pool.append([(r, 1) for r in running])

    def release(self, r):
        self.pool.free_seq(r)

    def held(self):
        return (self.N - self.pool.num_free()) * self.B

    def largest_free(self):
        return self.pool.num_free() * self.B  # any free block serves any request


class _ContiguousMemory:
    def __init__(self, capacity, reserve):
        self.capacity = capacity
        self.reserve = reserve
        self.holes = [[0, capacity]] if capacity else []  # [offset, size], by offset
        self.where = {}

    def need(self, r, tokens):
        return self.reserve[r]

    def admit(self, r, tokens):
        R = self.reserve[r]
        for h in self.holes:  # first fit: the lowest-addressed hole that is large enough
            if h[1] >= R:
                self.where[r] = (h[0], R)
                h[0] += R
                h[1] -= R
                if h[1] == 0:
                    self.holes.remove(h)
                return True
        return False

    def grow(self, running):
        pass  # the reservation already covers the request's final length

    def release(self, r):
        off, size = self.where.pop(r)
        self.holes.append([off, size])
        self.holes.sort()
        merged = []
        for h in self.holes:
            if merged and merged[-1][0] + merged[-1][1] == h[0]:
                merged[-1][1] += h[1]
            else:
                merged.append(h)
        self.holes = merged

    def held(self):
        return sum(size for _, size in self.where.values())

    def largest_free(self):
        return max((h[1] for h in self.holes), default=0)


def _run(mem, capacity, max_batch, arrival, prompt, output, max_steps):
    n = len(arrival)
    g = [0] * n
    finish = [-1] * n
    waiting = deque()
    running = []  # admission order: the last is the newest
    rows = []
    nxt = 0
    t = 0
    while True:
        if t >= max_steps:
            raise Stalled(f"requests still running or waiting after {max_steps} steps")
        while nxt < n and arrival[nxt] == t:
            waiting.append(nxt)
            nxt += 1
        preempted = 0
        while running:
            try:
                mem.grow(running)
                break
            except OutOfBlocks:
                victim = running.pop()
                mem.release(victim)
                waiting.appendleft(victim)
                preempted += 1
        for r in running:
            g[r] += 1
        decoded = len(running)
        done = [r for r in running if g[r] == output[r]]
        for r in done:
            mem.release(r)
            finish[r] = t
        running = [r for r in running if g[r] < output[r]]
        admitted = blocked = 0
        while waiting and len(running) < max_batch:
            h = waiting[0]
            if not mem.admit(h, prompt[h] + g[h]):
                blocked = mem.need(h, prompt[h] + g[h])
                break
            waiting.popleft()
            running.append(h)
            admitted += 1
        held = mem.held()
        rows.append((t, len(running), len(waiting), sum(prompt[r] + g[r] for r in running), held, capacity - held,
                     mem.largest_free(), admitted, preempted, len(done), decoded, blocked,
                     sum(prompt[r] + output[r] for r in running)))
        t += 1
        if nxt == n and not waiting and not running:
            return rows, finish


def _check_requests(arrival, prompt, output):
    if not (len(arrival) == len(prompt) == len(output)):
        raise ValueError("arrival, prompt and output differ in length")
    if any(a < 0 for a in arrival) or any(b < a for a, b in zip(arrival, arrival[1:])):
        raise ValueError("arrival steps must be >= 0 and non-decreasing")
    if any(p < 1 for p in prompt) or any(o < 1 for o in output):
        raise ValueError("prompt and output lengths must be >= 1")


def simulate_paged(num_blocks, block_size, watermark, max_batch, arrival, prompt, output, max_steps=10 ** 7):
    """Paged scheme over a pool of num_blocks blocks of block_size slots. Returns (rows, finish):
    one tuple per step in FIELDS order, and the step each request finished at."""
    arrival, prompt, output = ([int(x) for x in a] for a in (arrival, prompt, output))
    _check_requests(arrival, prompt, output)
    if num_blocks <= 0 or block_size <= 0 or watermark < 0 or max_batch <= 0:
        raise ValueError("num_blocks, block_size and max_batch must be positive, watermark >= 0")
    for p, o in zip(prompt, output):
        if -(-(p + o) // block_size) + watermark > num_blocks:
            raise ValueError("a request can never fit in the pool")
    return _run(_PagedMemory(num_blocks, block_size, watermark), num_blocks * block_size, max_batch,
                arrival, prompt, output, max_steps)


def simulate_contiguous(capacity, max_batch, arrival, prompt, output, reserve, max_steps=10 ** 7):
    """Contiguous-reservation scheme over capacity slots; request i reserves reserve[i] >= P + O
    slots. Returns (rows, finish) as simulate_paged."""
    arrival, prompt, output, reserve = ([int(x) for x in a] for a in (arrival, prompt, output, reserve))
    _check_requests(arrival, prompt, output)
    if len(reserve) != len(arrival):
        raise ValueError("reserve differs in length")
    if capacity <= 0 or max_batch <= 0:
        raise ValueError("capacity and max_batch must be positive")
    for p, o, R in zip(prompt, output, reserve):
        if R < p + o or R > capacity:
            raise ValueError("each reservation must cover P + O and fit the capacity")
    return _run(_ContiguousMemory(capacity, reserve), capacity, max_batch, arrival, prompt, output, max_steps)
