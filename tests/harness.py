"""Helpers shared by the GPU parity tests: replay a workload on both sides and compare."""
import sys
from functools import lru_cache

import numpy as np
import torch

import oracle
import synth
from paged_kv_cache_416_amd import kernels
from paged_kv_cache_416_amd.cache import PagedKVCache, run_ops, to_device

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# |gpu - ref64| <= ATOL + RTOL * |ref64|: 2e-3 for 16-bit storage, 1e-5 for fp32
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half a unit in the last place of bfloat16 at |ref| (normal range): the most that rounding a
    value of that binade to bf16 storage can move it. bf16 keeps 8 significant bits, so this is
    2^(e - 8) for |ref| in [2^e, 2^(e+1)): between 2^-9 and 2^-8 of |ref|."""
    e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-30)))
    return np.exp2(e - 8)


def assert_close(got: torch.Tensor, ref: np.ndarray, dtype: str, what="", bf16_storage=False):
    """|gpu - ref| <= tol + tol*|ref| element by element. With bf16_storage (bf16 outputs only),
    plus half a bf16 ulp at |ref|: storing an output in bf16 alone can err by up to 2^-8 |o|, which
    is above tol + tol*|o| once |o| exceeds about 1.05. For f16 (2^-11 |o|) and fp32 storage
    never needs an allowance, so they always take the plain bound."""
    g = to_f64(got)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert not bf16_storage or dtype == "bf16", "the storage allowance is for bf16 outputs only"
    tol = TOL[dtype]
    err = np.abs(g - ref)
    bound = tol + tol * np.abs(ref)
    if bf16_storage:
        bound = bound + bf16_half_ulp(ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), ref.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} outside tolerance; worst at {i}: "
                             f"gpu={g[i]!r} ref={ref[i]!r} err={err[i]:.3e}")
    return float(err.max(initial=0.0))


def worst_margin(got: torch.Tensor, ref: np.ndarray, dtype: str) -> float:
    """max over elements of |gpu - ref| / (tol + tol*|ref|): below 1 inside the plain bound."""
    tol = TOL[dtype]
    return float((np.abs(to_f64(got) - ref) / (tol + tol * np.abs(ref))).max(initial=0.0))


def cache_bytes(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


def same_bytes(a: np.ndarray, b: np.ndarray, what="") -> bool:
    """Byte equality of two flat uint8 arrays; on mismatch raise with the first differing offset."""
    if a.shape != b.shape:
        raise AssertionError(f"{what}: {a.shape} bytes vs {b.shape}")
    diff = np.flatnonzero(a != b)
    if diff.size:
        i = int(diff[0])
        raise AssertionError(f"{what}: {diff.size} bytes differ, first at offset {i}: {a[i]} vs {b[i]}")
    return True


def host_bytes(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


def gpu_replay(w, on_check=None):
    dt = TORCH_DTYPE[w.dtype]
    c = PagedKVCache(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, dt, free_order=w.free_order)
    run_ops(c, w.ops, dt, on_check=(lambda: on_check(c)) if on_check else None)
    torch.cuda.synchronize()
    return c


def gpu_attention(c, w, partition_size=None, flags=0, q=None, cached_lens=None):
    dt = TORCH_DTYPE[w.dtype]
    qd = to_device(w.q, dt, c.device) if q is None else q
    P = w.partition_size if partition_size is None else partition_size
    out = c.attention(qd, w.batch, w.scale, partition_size=P, flags=flags, cached_lens=cached_lens)
    torch.cuda.synchronize()
    return out


@lru_cache(maxsize=4)
def oracle_state(key, builder, *args):
    """Oracle replay, cached by key (workloads are deterministic)."""
    w = builder(*args)
    return w, oracle.replay(w)
