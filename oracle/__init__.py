"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library (``paged_kv_cache_416_amd``)
never imports it, and this package imports nothing from the GPU library: the
two share only the seeded inputs of ``synth``.

Contents
  * ``liboracle.so`` (``oracle.c``): byte-level cache writes and block copies,
    and attention in double precision, gathered through the block table
    ("vLLM and PagedAttention" slides, slide 9 and slide 11; "Week 22 Day 2"
    lesson note, section 2).
  * ``allocator.BlockPool``: the allocator model (slides 10-15; lesson note
    sections 2-4).
  * ``replay``: runs a workload's operations with the two pieces above.

Every function here has a pin in ``tests/test_oracle_*.py`` that does not go
through this package's own formulas (library routines, closed forms, the
pages' worked examples, invariants).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

from .allocator import BlockPool, OutOfBlocks  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
_STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}
_ELT = {"f32": 4, "f16": 2, "bf16": 2}

_p = ctypes.c_void_p
_i32, _i64, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from .build import build
            build()
        L = ctypes.CDLL(path)
        L.oracle_decode_element.argtypes = [_p, _p, _i64, ctypes.c_int]
        L.oracle_reshape_and_cache.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _i32, _i32, _i32, _i32, _i32]
        L.oracle_copy_blocks.argtypes = [_p, _p, _i64, _i64, _p, _i32]
        L.oracle_paged_attention.argtypes = [_p, _p, _p, _p, _i64, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32,
                                             _f64, _i32, _i32]
        L.oracle_contiguous_attention.argtypes = [_p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _f64, _i32]
        L.oracle_paged_prefill.argtypes = [_p, _p, _p, _p, _i64, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                           _f64, _i32]
        for f in (L.oracle_decode_element, L.oracle_reshape_and_cache, L.oracle_copy_blocks,
                  L.oracle_paged_attention, L.oracle_contiguous_attention, L.oracle_paged_prefill, L.oracle_threads):
            f.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _raw(a, dtype):
    """View a storage array (float32 / float16 / uint16-bits) as the oracle's raw element type."""
    a = np.ascontiguousarray(a)
    return a.view(_STORAGE[dtype]) if dtype != "f32" else a.astype(np.float32, copy=False)


def threads():
    return lib().oracle_threads()


def decode(a, dtype):
    """Widen storage elements to float64 with the oracle's own binary16 / bf16 decoders."""
    src = _raw(a, dtype)
    out = np.empty(src.shape, np.float64)
    rc = lib().oracle_decode_element(_ptr(out), _ptr(src), src.size, DTYPE_CODE[dtype])
    assert rc == 0
    return out


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, block_size):
    """key/value [T, Hkv, D]; caches [N, Hkv, B, D] (modified in place); slot < 0 is skipped."""
    assert key.shape == value.shape and key.ndim == 3
    T, hkv, d = key.shape
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    assert slots.shape == (T,)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    rc = lib().oracle_reshape_and_cache(_ptr(key), _ptr(value), hkv * d, hkv * d, _ptr(k_cache), _ptr(v_cache),
                                        k_cache.shape[0], _ptr(slots), T, hkv, d, block_size,
                                        key.itemsize)
    if rc:
        raise ValueError("oracle_reshape_and_cache: invalid slot")


def copy_blocks(k_cache, v_cache, pairs):
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    block_bytes = k_cache[0].nbytes
    rc = lib().oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), k_cache.shape[0], block_bytes, _ptr(pairs),
                                  pairs.shape[0])
    if rc:
        raise ValueError("oracle_copy_blocks: block out of range")


def paged_attention(q, k_cache, v_cache, tables, ctx, scale, dtype, partition_size=0):
    """q [S, Hq, D]; caches [N, Hkv, B, D]; tables int32 [S, max_blocks]; ctx int32 [S] -> float64 [S, Hq, D]."""
    S, hq, d = q.shape
    N, hkv, B, d2 = k_cache.shape
    assert d == d2
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    out = np.zeros((S, hq, d), np.float64)
    qr, kr, vr = _raw(q, dtype), _raw(k_cache, dtype), _raw(v_cache, dtype)
    rc = lib().oracle_paged_attention(_ptr(out), _ptr(qr), _ptr(kr), _ptr(vr), N, _ptr(tables),
                                      tables.shape[1] if tables.ndim == 2 else 0, _ptr(ctx), S, hq, hkv, d, B,
                                      float(scale), int(partition_size), DTYPE_CODE[dtype])
    if rc:
        raise ValueError(f"oracle_paged_attention failed ({rc})")
    return out


def paged_prefill(q, k_cache, v_cache, tables, ctx, query_start, scale, dtype):
    """q [T, Hq, D] (rows query_start[s]..query_start[s+1]-1 are sequence s's last queries, causal
    over its ctx[s] keys); caches [N, Hkv, B, D]; tables int32 [S, max_blocks] -> float64 [T, Hq, D]."""
    T, hq, d = q.shape
    N, hkv, B, d2 = k_cache.shape
    assert d == d2
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    assert qs[-1] == T
    out = np.zeros((T, hq, d), np.float64)
    qr, kr, vr = _raw(q, dtype), _raw(k_cache, dtype), _raw(v_cache, dtype)
    rc = lib().oracle_paged_prefill(_ptr(out), _ptr(qr), _ptr(kr), _ptr(vr), N, _ptr(tables),
                                    tables.shape[1] if tables.ndim == 2 else 0, _ptr(ctx), _ptr(qs), len(ctx), hq,
                                    hkv, d, B, float(scale), DTYPE_CODE[dtype])
    if rc:
        raise ValueError(f"oracle_paged_prefill failed ({rc})")
    return out


def contiguous_attention(q, k, v, ctx, scale, dtype):
    """q [S, Hq, D]; k, v [S, Hkv, Lmax, D]; ctx int32 [S] -> float64 [S, Hq, D]."""
    S, hq, d = q.shape
    _, hkv, lmax, _ = k.shape
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    out = np.zeros((S, hq, d), np.float64)
    rc = lib().oracle_contiguous_attention(_ptr(out), _ptr(_raw(q, dtype)), _ptr(_raw(k, dtype)),
                                           _ptr(_raw(v, dtype)), lmax, _ptr(ctx), S, hq, hkv, d, float(scale),
                                           DTYPE_CODE[dtype])
    if rc:
        raise ValueError(f"oracle_contiguous_attention failed ({rc})")
    return out


# bit pattern used to poison cache memory that no token has been written to
POISON = {"f32": np.uint32(0x7FC00000), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


def poisoned_cache(num_blocks, num_kv_heads, block_size, head_dim, dtype):
    """A cache whose every element is a quiet NaN, so a read of an unwritten slot shows up in results."""
    raw = np.full((num_blocks, num_kv_heads, block_size, head_dim), POISON[dtype])
    if dtype == "f32":
        return raw.view(np.float32)
    if dtype == "f16":
        return raw.view(np.float16)
    return raw


@dataclass
class OracleState:
    pool: BlockPool
    k_cache: np.ndarray
    v_cache: np.ndarray
    step_slots: list = field(default_factory=list)  # slots of each append op, in order
    step_pairs: list = field(default_factory=list)  # copy pairs of each append op, in order
    checks: list = field(default_factory=list)  # attention outputs at each ("check",) op
    cached_tokens: list = field(default_factory=list)  # prompt tokens found in the prefix cache, per prompt op


def batch_tables(pool, batch, pad=-1):
    """Block tables and context lengths of ``batch``: int32 [S, max_blocks], int32 [S]."""
    mb = max([len(pool.blocks(s)) for s in batch] + [1])
    rows, ctx = pool.tables(batch, mb, pad)
    return np.array(rows, dtype=np.int32).reshape(len(batch), mb), np.array(ctx, dtype=np.int32)


def replay(w, attend_checks=True, partition_size=None, after_op=None):
    """Run a workload's operations with the oracle's allocator model, scatter and copy.

    after_op(index, op, state), if given, is called after each operation."""
    pool = BlockPool(w.num_blocks, w.block_size, w.free_order)
    kc = poisoned_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.dtype)
    vc = poisoned_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.dtype)
    st = OracleState(pool=pool, k_cache=kc, v_cache=vc)
    for i, op in enumerate(w.ops):
        kind = op[0]
        if kind == "add":
            pool.add(op[1])
        elif kind == "fork":
            pool.fork(op[1], op[2])
        elif kind == "free":
            pool.free_seq(op[1])
        elif kind == "append":
            reqs = [(sid, k.shape[0]) for sid, k, _ in op[1]]
            slots, pairs = pool.append(reqs)
            if pairs:
                copy_blocks(kc, vc, pairs)
            keys = np.concatenate([k for _, k, _ in op[1]])
            vals = np.concatenate([v for _, _, v in op[1]])
            reshape_and_cache(keys, vals, kc, vc, np.array(slots, np.int64), w.block_size)
            st.step_slots.append(slots)
            st.step_pairs.append(pairs)
        elif kind == "prompt":
            slots, n_cached = pool.add_prompt(op[1], [int(t) for t in op[2]])
            reshape_and_cache(op[3], op[4], kc, vc, np.array(slots, np.int64), w.block_size)
            st.step_slots.append(slots)
            st.step_pairs.append([])
            st.cached_tokens.append(n_cached)
        elif kind == "check":
            if attend_checks:
                tb, ctx = batch_tables(pool, w.batch)
                st.checks.append(paged_attention(w.q, kc, vc, tb, ctx, w.scale, w.dtype,
                                                 w.partition_size if partition_size is None else partition_size))
        else:
            raise ValueError(kind)
        if after_op is not None:
            after_op(i, op, st)
    return st


def attention_of(st, w, partition_size=0):
    tb, ctx = batch_tables(st.pool, w.batch)
    return paged_attention(w.q, st.k_cache, st.v_cache, tb, ctx, w.scale, w.dtype, partition_size)
