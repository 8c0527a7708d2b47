"""Python handle on the native continuous-batching memory simulator (pkv_sim_* in include/pkv.h)."""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import check, load

FIELDS = ("step", "running", "waiting", "used", "held", "free", "largest_free", "admitted", "preempted",
          "finished", "decoded", "blocked_need", "final_sum")

_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)


def _requests(arrival, prompt, output):
    a, p, o = (np.ascontiguousarray(x, dtype=np.int32) for x in (arrival, prompt, output))
    if not (a.ndim == p.ndim == o.ndim == 1 and len(a) == len(p) == len(o)):
        raise ValueError("arrival, prompt and output must be 1-D of one length")
    return a, p, o


def _outputs(n, max_steps):
    return np.empty((max_steps, len(FIELDS)), np.int64), np.empty(max(n, 1), np.int64), ctypes.c_int64()


def simulate_paged(num_blocks, block_size, watermark, max_batch, arrival, prompt, output, max_steps=1 << 16):
    """Paged scheme over this library's block pool. Returns (trace [steps, FIELDS], finish)."""
    a, p, o = _requests(arrival, prompt, output)
    trace, fin, steps = _outputs(len(a), max_steps)
    check(load().pkv_sim_paged(num_blocks, block_size, watermark, max_batch, a.ctypes.data_as(_pi32),
                               p.ctypes.data_as(_pi32), o.ctypes.data_as(_pi32), len(a), max_steps,
                               trace.ctypes.data_as(_pi64), ctypes.byref(steps), fin.ctypes.data_as(_pi64)))
    return trace[:steps.value].copy(), fin[:len(a)].copy()


def simulate_contiguous(capacity, max_batch, arrival, prompt, output, reserve, max_steps=1 << 16):
    """Contiguous first-fit reservations of reserve[i] slots. Returns (trace, finish)."""
    a, p, o = _requests(arrival, prompt, output)
    r = np.ascontiguousarray(reserve, dtype=np.int32)
    if r.shape != a.shape:
        raise ValueError("reserve must match the requests")
    trace, fin, steps = _outputs(len(a), max_steps)
    check(load().pkv_sim_contiguous(capacity, max_batch, a.ctypes.data_as(_pi32), p.ctypes.data_as(_pi32),
                                    o.ctypes.data_as(_pi32), r.ctypes.data_as(_pi32), len(a), max_steps,
                                    trace.ctypes.data_as(_pi64), ctypes.byref(steps), fin.ctypes.data_as(_pi64)))
    return trace[:steps.value].copy(), fin[:len(a)].copy()


def summarize(trace, capacity):
    """Figures of one run: the share of held slots that hold a real token (useful KV memory,
    slide 7) over all steps and over the steps with requests waiting (the saturated regime),
    the share of the whole capacity in use, mean batch, steps, evictions."""
    t = np.asarray(trace, dtype=np.int64)
    i = {n: k for k, n in enumerate(FIELDS)}
    sat = t[:, i["waiting"]] > 0

    def frac(mask):
        held = t[mask, i["held"]].sum()
        return float(t[mask, i["used"]].sum() / held) if held else None

    return {
        "steps": int(len(t)),
        "useful_of_held": frac(slice(None)),
        "useful_of_held_saturated": frac(sat),
        "useful_of_capacity_saturated": float(t[sat, i["used"]].sum() / (capacity * sat.sum())) if sat.any() else None,
        "mean_batch": float(t[:, i["running"]].mean()),
        "mean_batch_saturated": float(t[sat, i["running"]].mean()) if sat.any() else None,
        "evictions": int(t[:, i["preempted"]].sum()),
        "decoded": int(t[:, i["decoded"]].sum()),
    }
