"""Torch-tensor wrappers of the device entry points. Argument marshalling only: every step runs in libpkv.so.

Tensors must live on the current HIP device; kernels are enqueued on torch's current stream.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import PKV_BF16, PKV_F16, PKV_F32, check, load

_DTYPE = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}


def dtype_code(t: torch.dtype) -> int:
    try:
        return _DTYPE[t]
    except KeyError:
        raise TypeError(f"unsupported dtype {t}") from None


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensor is not on a HIP device")


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """key/value [T, Hkv, D] (rows may be strided); caches [N, Hkv, B, D]; slot_mapping int64 [T] (device)."""
    _need_cuda(key, value, k_cache, v_cache, slot_mapping)
    T, hkv, d = key.shape
    if value.shape != key.shape or key.dtype != k_cache.dtype or value.dtype != k_cache.dtype:
        raise ValueError("key/value shape or dtype mismatch")
    if key.stride(2) != 1 or key.stride(1) != d or value.stride(2) != 1 or value.stride(1) != d:
        raise ValueError("key/value heads must be contiguous within a token row")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,) or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 [T] tensor")
    N, hkv2, B, d2 = k_cache.shape
    if (hkv2, d2) != (hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape mismatch")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    check(load().pkv_reshape_and_cache(_ptr(key), _ptr(value), key.stride(0), value.stride(0), _ptr(k_cache),
                                       _ptr(v_cache), N, _ptr(slot_mapping), T, hkv, d, B,
                                       dtype_code(k_cache.dtype), _stream()))


def copy_blocks(k_caches, v_caches, pairs):
    """Copy-on-write block copies in every layer. pairs: host (src, dst) pairs, e.g. from Pool.append."""
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    if pairs.shape[0] == 0:
        return
    L = len(k_caches)
    if len(v_caches) != L or L == 0:
        raise ValueError("need one K and one V cache per layer")
    _need_cuda(*k_caches, *v_caches)
    N = k_caches[0].shape[0]
    bb = k_caches[0][0].numel() * k_caches[0].element_size()
    for c in list(k_caches) + list(v_caches):
        if c.shape != k_caches[0].shape or not c.is_contiguous():
            raise ValueError("caches must be contiguous and of one shape")
    kp = (ctypes.c_void_p * L)(*[c.data_ptr() for c in k_caches])
    vp = (ctypes.c_void_p * L)(*[c.data_ptr() for c in v_caches])
    check(load().pkv_copy_blocks(kp, vp, L, N, bb, pairs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 pairs.shape[0], _stream()))


def swap_blocks(src_caches, dst_caches, pairs):
    """Copy blocks between two pools' caches (swap out / swap in). src_caches, dst_caches: lists of
    contiguous tensors [N_src, ...] / [N_dst, ...] of one block shape, each on the device or in
    pinned host memory; pairs: host (src block, dst block) pairs, e.g. from Pool.migrate."""
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    if pairs.shape[0] == 0:
        return
    C = len(src_caches)
    if len(dst_caches) != C or C == 0:
        raise ValueError("need one destination cache per source cache")
    for t in list(src_caches) + list(dst_caches):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError("caches must be device tensors or pinned host tensors")
        if not t.is_contiguous() or t.shape[1:] != src_caches[0].shape[1:] or t.dtype != src_caches[0].dtype:
            raise ValueError("caches must be contiguous, of one block shape and dtype")
    bb = src_caches[0][0].numel() * src_caches[0].element_size()
    sp = (ctypes.c_void_p * C)(*[t.data_ptr() for t in src_caches])
    dp = (ctypes.c_void_p * C)(*[t.data_ptr() for t in dst_caches])
    check(load().pkv_swap_blocks(sp, dp, C, src_caches[0].shape[0], dst_caches[0].shape[0], bb,
                                 pairs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), pairs.shape[0], _stream()))


def decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_size):
    return int(load().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_size))


def alloc_workspace(num_seqs, num_q_heads, head_dim, max_context_len, partition_size, device=None):
    n = decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_size)
    if n == 0:
        return None
    return torch.empty(n // 4, dtype=torch.float32, device=device or torch.device("cuda"))


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                           partition_size=0, workspace=None, flags=0, cached_lens=None):
    """out/q [S, Hq, D]; caches [N, Hkv, B, D]; block_tables int32 [S, max_blocks]; context_lens int32 [S];
    cached_lens: None or int32 [S], the load-policy hint (tokens per sequence in shared blocks)."""
    _need_cuda(out, q, k_cache, v_cache, block_tables, context_lens, workspace, cached_lens)
    S, hq, d = q.shape
    N, hkv, B, d2 = k_cache.shape
    if out.shape != q.shape or d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    for t in (out, q, k_cache, v_cache, block_tables, context_lens):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if q.dtype != k_cache.dtype or out.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("dtype mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    if cached_lens is not None and (cached_lens.dtype != torch.int32 or cached_lens.shape != (S,)
                                    or not cached_lens.is_contiguous()):
        raise ValueError("cached_lens must be a contiguous int32 [S]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(load().pkv_paged_attention_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), N, _ptr(block_tables),
                                            block_tables.shape[1], _ptr(context_lens), int(max_context_len), S, hq,
                                            hkv, d, B, float(scale), int(partition_size), _ptr(workspace), ws_bytes,
                                            dtype_code(q.dtype), int(flags), _ptr(cached_lens), _stream()))
    return out


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                                   partition_size=0, flags=0, cached_lens=None):
    """paged_attention_decode with no workspace argument: a split takes its workspace from the library's
    static per-device array (for callers that cannot allocate). Calls on one device must not overlap."""
    _need_cuda(out, q, k_cache, v_cache, block_tables, context_lens, cached_lens)
    S, hq, d = q.shape
    N, hkv, B, d2 = k_cache.shape
    if out.shape != q.shape or d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    for t in (out, q, k_cache, v_cache, block_tables, context_lens):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if q.dtype != k_cache.dtype or out.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("dtype mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    if cached_lens is not None and (cached_lens.dtype != torch.int32 or cached_lens.shape != (S,)
                                    or not cached_lens.is_contiguous()):
        raise ValueError("cached_lens must be a contiguous int32 [S]")
    check(load().pkv_paged_attention_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), N,
                                                    _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                                    int(max_context_len), S, hq, hkv, d, B, float(scale),
                                                    int(partition_size), dtype_code(q.dtype), int(flags),
                                                    _ptr(cached_lens), _stream()))
    return out


def paged_attention_decode_step(out, q, new_k, new_v, slot_mapping, k_cache, v_cache, block_tables, context_lens,
                                max_context_len, scale, partition_size=0, workspace=None, flags=0, cached_lens=None):
    """reshape_and_cache(new_k, new_v, slot_mapping) then paged_attention_decode, in one launch.
    new_k/new_v [S, Hkv, D] (sequence s's token at position context_lens[s] - 1); slot_mapping int64 [S]."""
    _need_cuda(out, q, new_k, new_v, slot_mapping, k_cache, v_cache, block_tables, context_lens, workspace,
               cached_lens)
    S, hq, d = q.shape
    N, hkv, B, d2 = k_cache.shape
    if out.shape != q.shape or d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if new_k.shape != (S, hkv, d) or new_v.shape != new_k.shape or slot_mapping.shape != (S,):
        raise ValueError("new_k/new_v must be [S, Hkv, D] and slot_mapping [S]")
    for t in (out, q, new_k, new_v, slot_mapping, k_cache, v_cache, block_tables, context_lens):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if len({t.dtype for t in (out, q, new_k, new_v, k_cache, v_cache)}) != 1:
        raise ValueError("dtype mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or slot_mapping.dtype != torch.int64:
        raise ValueError("block_tables and context_lens must be int32, slot_mapping int64")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    if cached_lens is not None and (cached_lens.dtype != torch.int32 or cached_lens.shape != (S,)
                                    or not cached_lens.is_contiguous()):
        raise ValueError("cached_lens must be a contiguous int32 [S]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(load().pkv_paged_attention_decode_step(_ptr(out), _ptr(q), _ptr(new_k), _ptr(new_v), _ptr(slot_mapping),
                                                 _ptr(k_cache), _ptr(v_cache), N, _ptr(block_tables),
                                                 block_tables.shape[1], _ptr(context_lens), int(max_context_len), S,
                                                 hq, hkv, d, B, float(scale), int(partition_size), _ptr(workspace),
                                                 ws_bytes, dtype_code(q.dtype), int(flags), _ptr(cached_lens),
                                                 _stream()))
    return out


def contiguous_attention_decode(out, q, k, v, context_lens, max_context_len, scale, partition_size=0,
                                workspace=None, flags=0):
    """out/q [S, Hq, D]; k, v [S, Hkv, Lmax, D]; context_lens int32 [S]."""
    _need_cuda(out, q, k, v, context_lens, workspace)
    S, hq, d = q.shape
    S2, hkv, lmax, d2 = k.shape
    if out.shape != q.shape or S2 != S or d2 != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    for t in (out, q, k, v, context_lens):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if q.dtype != k.dtype or out.dtype != q.dtype or v.dtype != q.dtype or context_lens.dtype != torch.int32:
        raise ValueError("dtype mismatch")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(load().pkv_contiguous_attention_decode(_ptr(out), _ptr(q), _ptr(k), _ptr(v), lmax, _ptr(context_lens),
                                                 int(max_context_len), S, hq, hkv, d, float(scale),
                                                 int(partition_size), _ptr(workspace), ws_bytes,
                                                 dtype_code(q.dtype), int(flags), _stream()))
    return out


def read_probe(src, sink):
    """Read all of src (a contiguous device tensor, size a multiple of 16 bytes) once; sink is a
    device tensor of at least 4 bytes (the probe's liveness sink)."""
    _need_cuda(src, sink)
    if not src.is_contiguous() or sink.numel() * sink.element_size() < 4:
        raise ValueError("src must be contiguous and sink at least 4 bytes")
    check(load().pkv_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream()))


def paged_attention_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len,
                            max_context_len, scale, flags=0):
    """out/q [T, Hq, D] (rows query_start[s]..query_start[s+1]-1 are sequence s's last queries, causal);
    caches [N, Hkv, B, D]; block_tables int32 [S, max_blocks]; context_lens int32 [S]; query_start int32 [S+1]
    with query_start[S] <= T (the library bounds the rows by T on the device)."""
    T, hq, d = q.shape
    N, hkv, B, d2 = k_cache.shape
    S = context_lens.shape[0]
    if out.shape != q.shape or d2 != d or v_cache.shape != k_cache.shape or query_start.shape != (S + 1,):
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError(f"block_tables must be [S={S}, max_blocks], got {tuple(block_tables.shape)}")
    _need_cuda(out, q, k_cache, v_cache, block_tables, context_lens, query_start)
    for t in (out, q, k_cache, v_cache, block_tables, context_lens, query_start):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if q.dtype != k_cache.dtype or out.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("dtype mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or query_start.dtype != torch.int32:
        raise ValueError("tables, lengths and query_start must be int32")
    check(load().pkv_paged_attention_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), N, _ptr(block_tables),
                                             block_tables.shape[1], _ptr(context_lens), _ptr(query_start), T,
                                             int(max_query_len), int(max_context_len), S, hq, hkv, d, B, float(scale),
                                             dtype_code(q.dtype), int(flags), _stream()))
    return out
