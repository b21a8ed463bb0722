"""pkv: paged KV cache and paged attention for AMD Instinct MI355X (gfx950).

A thin binding of libpkv's C ABI (``include/pkv.h``): every function here
carries the C name, checks and marshals its arguments (torch tensors for
device memory, numpy arrays for host memory, torch's current HIP stream) and
calls the library.  All work happens in the library: the host block manager
in C++ and every device step in hand-written gfx950 HIP kernels.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence, Tuple

import numpy as np

from ._lib import (PKV_ALGO_AUTO, PKV_ALGO_MFMA, PKV_ALGO_WAVE, PKV_BF16, PKV_ERR_DEVICE,  # noqa
                   PKV_ERR_INTERNAL, PKV_ERR_INVALID, PKV_ERR_OUT_OF_BLOCKS, PKV_ERR_UNSUPPORTED,
                   PKV_F16, PKV_F32, PKV_I4, PKV_I8, PKV_KV_CACHED, PKV_KV_STREAM,
                   PKV_MERGE_IN_KERNEL, PKV_NOALLOC_SCRATCH_BYTES, PKV_OK, LIB_PATH,
                   PkvBmLatency, PkvBmStats, PkvError, PkvSwapStats, PkvOutOfBlocks, check, load)

__all__ = [n for n in dir() if n.startswith("pkv_") or n.startswith("PKV_")]


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int32))


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int64))


# --------------------------------------------------------------------------
# host block manager
# --------------------------------------------------------------------------
def pkv_version() -> str:
    return load().pkv_version().decode()


def pkv_bm_create(num_blocks: int, block_size: int,
                  init_free_order: Optional[Sequence[int]] = None) -> C.c_void_p:
    h = C.c_void_p()
    order = None
    if init_free_order is not None:
        order = np.ascontiguousarray(init_free_order, dtype=np.int32)
        if order.shape != (num_blocks,):
            raise ValueError("init_free_order must have num_blocks entries")
    check(load().pkv_bm_create(num_blocks, block_size, _i32p(order) if order is not None else None,
                               C.byref(h)))
    return h


def pkv_bm_destroy(bm) -> None:
    load().pkv_bm_destroy(bm)


def pkv_bm_alloc(bm, n: int) -> np.ndarray:
    ids = np.empty(max(n, 0), np.int32)
    check(load().pkv_bm_alloc(bm, n, _i32p(ids)))
    return ids


def pkv_bm_incref(bm, block: int) -> None:
    check(load().pkv_bm_incref(bm, block))


def pkv_bm_decref(bm, block: int) -> None:
    check(load().pkv_bm_decref(bm, block))


def pkv_bm_num_free(bm) -> int:
    return load().pkv_bm_num_free(bm)


def pkv_bm_get_state(bm, num_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
    free = np.empty(num_blocks, np.int32)
    rc = np.empty(num_blocks, np.int32)
    n = C.c_int32()
    check(load().pkv_bm_get_state(bm, _i32p(free), C.byref(n), _i32p(rc)))
    return free[:n.value].copy(), rc


def pkv_bm_stats_get(bm) -> dict:
    s = PkvBmStats()
    check(load().pkv_bm_stats_get(bm, C.byref(s)))
    return {f: getattr(s, f) for f, _ in PkvBmStats._fields_}


def pkv_bm_latency_get(bm, reset: bool = False) -> dict:
    """Host latency of the block manager's allocating calls: count, window,
    p50 / p99 / max in microseconds."""
    st = PkvBmLatency()
    check(load().pkv_bm_latency_get(bm, C.byref(st), int(bool(reset))))
    return {name: getattr(st, name) for name, _ in st._fields_}


def pkv_seq_create(bm, num_tokens: int) -> int:
    sid = C.c_int64()
    check(load().pkv_seq_create(bm, num_tokens, C.byref(sid)))
    return sid.value


def pkv_seq_fork(bm, parent: int) -> int:
    sid = C.c_int64()
    check(load().pkv_seq_fork(bm, parent, C.byref(sid)))
    return sid.value


def pkv_seq_append(bm, seq: int, num_tokens: int = 1):
    """Returns (slots int32[num_tokens], (cow_src, cow_dst) or None)."""
    slots = np.empty(max(num_tokens, 0), np.int32)
    src, dst = C.c_int32(-1), C.c_int32(-1)
    check(load().pkv_seq_append(bm, seq, num_tokens, _i32p(slots), C.byref(src), C.byref(dst)))
    return slots, ((src.value, dst.value) if src.value >= 0 else None)


def pkv_seq_append_batch(bm, seqs: Sequence[int]):
    """Returns (slots int32[n], cow pairs int32[k, 2])."""
    s = np.ascontiguousarray(seqs, dtype=np.int64)
    slots = np.empty(len(s), np.int32)
    pairs = np.empty((max(len(s), 1), 2), np.int32)
    k = C.c_int32(0)
    check(load().pkv_seq_append_batch(bm, _i64p(s), len(s), _i32p(slots), _i32p(pairs),
                                      C.byref(k)))
    return slots, pairs[:k.value].copy()


def pkv_seq_slots(bm, seq: int, start: int, count: int) -> np.ndarray:
    out = np.empty(max(count, 0), np.int32)
    check(load().pkv_seq_slots(bm, seq, start, count, _i32p(out)))
    return out


def pkv_seq_len(bm, seq: int) -> int:
    n = C.c_int32()
    check(load().pkv_seq_len(bm, seq, C.byref(n)))
    return n.value


def pkv_seq_free(bm, seq: int) -> None:
    check(load().pkv_seq_free(bm, seq))


def pkv_seq_export(bm, seqs: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
    s = np.ascontiguousarray(seqs, dtype=np.int64)
    tables = np.empty((len(s), max_blocks), np.int32)
    lens = np.empty(len(s), np.int32)
    check(load().pkv_seq_export(bm, _i64p(s), len(s), max_blocks, _i32p(tables), _i32p(lens)))
    return tables, lens


def pkv_adaptive_block_size(avg_context_len: float) -> int:
    return load().pkv_adaptive_block_size(float(avg_context_len))


def pkv_seq_create_cached(bm, tokens) -> Tuple[int, int]:
    """Returns (sequence id, leading positions already cached)."""
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    sid, cached = C.c_int64(), C.c_int32()
    check(load().pkv_seq_create_cached(bm, _i32p(t), len(t), C.byref(sid), C.byref(cached)))
    return sid.value, cached.value


def pkv_seq_publish(bm, seq: int, tokens) -> int:
    """Index the sequence's full blocks under ``tokens``; returns the number
    of new entries."""
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    added = C.c_int32()
    check(load().pkv_seq_publish(bm, seq, _i32p(t), len(t), C.byref(added)))
    return added.value


def pkv_bm_prefix_stats(bm) -> dict:
    lookups, hits, cached = C.c_int64(), C.c_int64(), C.c_int32()
    check(load().pkv_bm_prefix_stats(bm, C.byref(lookups), C.byref(hits), C.byref(cached)))
    return {"cached_blocks": cached.value, "lookups": lookups.value, "hits": hits.value}


# --------------------------------------------------------------------------
# device operations (torch tensors on the GPU)
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    """Storage code of a tensor; uint8 tensors are 4-bit pools (two codes a byte)."""
    torch = _torch()
    m = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
         torch.int8: PKV_I8, torch.uint8: PKV_I4}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _pool_head_dim(pool) -> int:
    """head_dim of a pool [NB, Hkv, BS, D] (4-bit pools: [NB, Hkv, BS, D / 2] bytes)."""
    return pool.shape[3] * (2 if _dtype_code(pool) == PKV_I4 else 1)


def _dev(t, name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return C.c_void_p(t.data_ptr())


def _stream(t, stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return C.c_void_p(s.cuda_stream)


def pkv_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """key/value [T, Hkv, D] (row stride from the tensor), caches [NB, Hkv, BS, D]."""
    torch = _torch()
    T, hkv, d = key.shape
    nb, hkv2, bs, d2 = k_cache.shape
    if (hkv, d) != (hkv2, d2) or value.shape != key.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if key.dtype != k_cache.dtype or value.dtype != k_cache.dtype:
        raise TypeError("key, value and cache must share a dtype")
    for t, n in ((key, "key"), (value, "value")):
        if t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError(f"{n} rows must be [Hkv, D] contiguous")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    check(load().pkv_reshape_and_cache(
        C.c_void_p(key.data_ptr()), C.c_void_p(value.data_ptr()), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping", torch.int32), T,
        key.stride(0), value.stride(0), hkv, d, bs, nb, _dtype_code(k_cache),
        _stream(k_cache, stream)))


def _reshape_and_cache_codes(fn, code_dtype, key, value, k_codes, v_codes, k_scale, v_scale,
                             slot_mapping, stream):
    torch = _torch()
    T, hkv, d = key.shape
    nb, hkv2, bs, _ = k_codes.shape
    if k_codes.dtype != code_dtype or v_codes.dtype != code_dtype:
        raise TypeError(f"code pools must be {code_dtype}")
    d2 = _pool_head_dim(k_codes)
    if (hkv, d) != (hkv2, d2) or value.shape != key.shape or v_codes.shape != k_codes.shape:
        raise ValueError("shape mismatch")
    if k_scale.shape != (nb, hkv) or v_scale.shape != (nb, hkv):
        raise ValueError("scales must be [NB, Hkv]")
    for t, n in ((key, "key"), (value, "value")):
        if t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError(f"{n} rows must be [Hkv, D] contiguous")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    check(fn(
        C.c_void_p(key.data_ptr()), C.c_void_p(value.data_ptr()), _dtype_code(key),
        _dev(k_codes, "k_codes"), _dev(v_codes, "v_codes"), _dev(k_scale, "k_scale", torch.float32),
        _dev(v_scale, "v_scale", torch.float32), _dev(slot_mapping, "slot_mapping", torch.int32), T,
        key.stride(0), value.stride(0), hkv, d, bs, nb, _stream(k_codes, stream)))


def pkv_reshape_and_cache_int8(key, value, k_codes, v_codes, k_scale, v_scale, slot_mapping,
                               stream=None) -> None:
    """key/value [T, Hkv, D] (f32/f16/bf16, row stride from the tensor); int8
    pools [NB, Hkv, BS, D] and float32 scales [NB, Hkv]."""
    _reshape_and_cache_codes(load().pkv_reshape_and_cache_int8, _torch().int8, key, value,
                             k_codes, v_codes, k_scale, v_scale, slot_mapping, stream)


def pkv_reshape_and_cache_int4(key, value, k_codes, v_codes, k_scale, v_scale, slot_mapping,
                               stream=None) -> None:
    """key/value [T, Hkv, D] (f32/f16/bf16, row stride from the tensor); 4-bit
    pools uint8 [NB, Hkv, BS, D / 2] and float32 scales [NB, Hkv]."""
    _reshape_and_cache_codes(load().pkv_reshape_and_cache_int4, _torch().uint8, key, value,
                             k_codes, v_codes, k_scale, v_scale, slot_mapping, stream)


def pkv_copy_blocks(k_cache, v_cache, pairs, k_scale=None, v_scale=None, stream=None) -> None:
    """pairs: int32 [n, 2] device tensor of (src, dst)."""
    torch = _torch()
    nb, hkv, bs, _ = k_cache.shape
    d = _pool_head_dim(k_cache)
    n = pairs.shape[0] if pairs.dim() == 2 else 0
    check(load().pkv_copy_blocks(
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(k_scale, "k_scale", torch.float32),
        _dev(v_scale, "v_scale", torch.float32), _dev(pairs, "pairs", torch.int32), n, hkv, d, bs,
        nb, _dtype_code(k_cache), _stream(k_cache, stream)))


def pkv_swap_stats_get(reset: bool = False) -> dict:
    st = PkvSwapStats()
    check(load().pkv_swap_stats_get(C.byref(st), 1 if reset else 0))
    return {f: getattr(st, f) for f, _ in PkvSwapStats._fields_}


def pkv_swap_workspace_bytes(max_pairs: int, num_kv_heads: int, head_dim: int, block_size: int,
                             dtype_code: int) -> int:
    return load().pkv_swap_workspace_bytes(max_pairs, num_kv_heads, head_dim, block_size,
                                           dtype_code)


def pkv_swap_blocks(dst_k, dst_v, src_k, src_v, pairs, dst_k_scale=None, dst_v_scale=None,
                    src_k_scale=None, src_v_scale=None, workspace=None, stream=None) -> None:
    """Block d of the destination pools <- block s of the source pools for each
    (s, d) row of `pairs` (host int32 [n, 2]).  Pools are torch tensors
    [NB, Hkv, BS, D] on the GPU or in pinned host memory; `workspace` is an
    optional uint8 GPU tensor (see pkv_swap_workspace_bytes)."""
    torch = _torch()
    if dst_k.shape[1:] != src_k.shape[1:] or dst_v.shape != dst_k.shape or src_v.shape != src_k.shape:
        raise ValueError("pools must share [Hkv, BS, D]")
    if not (dst_k.dtype == dst_v.dtype == src_k.dtype == src_v.dtype):
        raise TypeError("pools must share a dtype")
    for t, n in ((dst_k, "dst_k"), (dst_v, "dst_v"), (src_k, "src_k"), (src_v, "src_v")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{n} must be a GPU tensor or pinned host memory")
    p = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    _, hkv, bs, _ = src_k.shape
    d = _pool_head_dim(src_k)
    ptr = lambda t: None if t is None else C.c_void_p(t.data_ptr())
    dev = dst_k if dst_k.is_cuda else src_k
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if workspace is not None and not workspace.is_cuda:
        raise ValueError("workspace must be a GPU tensor")
    check(load().pkv_swap_blocks(
        ptr(dst_k), ptr(dst_v), ptr(dst_k_scale), ptr(dst_v_scale), dst_k.shape[0], ptr(src_k),
        ptr(src_v), ptr(src_k_scale), ptr(src_v_scale), src_k.shape[0], _i32p(p), p.shape[0],
        hkv, d, bs, _dtype_code(src_k), ptr(workspace), ws_len, _stream(dev, stream)))


def _quantize_blocks(fn, code_dtype, src_k, src_v, dst_k, dst_v, k_scale, v_scale, blocks,
                     filled, stream):
    torch = _torch()
    nb, hkv, bs, d = src_k.shape
    if dst_k.dtype != code_dtype or dst_v.dtype != code_dtype:
        raise TypeError(f"code pools must be {code_dtype}")
    if (src_v.shape != src_k.shape or dst_v.shape != dst_k.shape
            or dst_k.shape[:3] != src_k.shape[:3] or _pool_head_dim(dst_k) != d):
        raise ValueError("pools must share one shape")
    if src_v.dtype != src_k.dtype:
        raise TypeError("src_k and src_v must share a dtype")
    if k_scale.shape != (nb, hkv) or v_scale.shape != (nb, hkv):
        raise ValueError("scales must be [num_blocks, num_kv_heads]")
    n = blocks.shape[0]
    if filled.shape != (n,):
        raise ValueError("blocks and filled must have one entry per listed block")
    check(fn(
        _dev(src_k, "src_k"), _dev(src_v, "src_v"), _dtype_code(src_k),
        _dev(dst_k, "dst_k", code_dtype), _dev(dst_v, "dst_v", code_dtype),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(blocks, "blocks", torch.int32), _dev(filled, "filled", torch.int32), n, hkv, d, bs,
        nb, _stream(src_k, stream)))


def pkv_quantize_blocks(src_k, src_v, dst_k, dst_v, k_scale, v_scale, blocks, filled,
                        stream=None) -> None:
    """src pools [NB, Hkv, BS, D] (f32/f16/bf16) -> int8 pools of the same shape
    and float32 scales [NB, Hkv], for the listed blocks (int32 [n] device
    tensors of block ids and filled row counts)."""
    _quantize_blocks(load().pkv_quantize_blocks, _torch().int8, src_k, src_v, dst_k, dst_v,
                     k_scale, v_scale, blocks, filled, stream)


def pkv_quantize_blocks_int4(src_k, src_v, dst_k, dst_v, k_scale, v_scale, blocks, filled,
                             stream=None) -> None:
    """src pools [NB, Hkv, BS, D] (f32/f16/bf16) -> 4-bit pools uint8
    [NB, Hkv, BS, D / 2] and float32 scales [NB, Hkv], for the listed blocks."""
    _quantize_blocks(load().pkv_quantize_blocks_int4, _torch().uint8, src_k, src_v, dst_k, dst_v,
                     k_scale, v_scale, blocks, filled, stream)


def pkv_decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int,
                               max_context_len: int, partition_tokens: int) -> int:
    return load().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                                             partition_tokens)


def pkv_decode_partition_for_capacity(context_lens, workgroups_per_partition: int,
                                      resident_workgroups: int, min_tokens: int) -> int:
    """Shortest partition whose workgroups fill the launch's whole rounds
    (0: no split); context_lens is a host sequence of lengths."""
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = C.c_int32(0)
    check(load().pkv_decode_partition_for_capacity(_i32p(lens), len(lens), workgroups_per_partition,
                                                   resident_workgroups, min_tokens, C.byref(out)))
    return out.value


def pkv_decode_partition_tokens(context_lens, q_dtype: int, kv_dtype: int, num_q_heads: int,
                                num_kv_heads: int, head_dim: int, block_size: int,
                                num_blocks: int, algo: int = PKV_ALGO_AUTO) -> int:
    """Partition for the decode kernel these arguments launch on the current
    device (0: no split); context_lens is a host sequence of lengths."""
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = C.c_int32(0)
    check(load().pkv_decode_partition_tokens(_i32p(lens), len(lens), q_dtype, kv_dtype, num_q_heads,
                                             num_kv_heads, head_dim, block_size, num_blocks, algo,
                                             C.byref(out)))
    return out.value


def pkv_prefill_partition_tokens(query_lens, context_lens, num_q_heads: int,
                                 q_dtype: int = PKV_BF16) -> int:
    """Key partition for a chunked-prefill launch on the current device (0:
    no split); query_lens and context_lens are host sequences of lengths."""
    ql = np.ascontiguousarray(query_lens, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    if ql.shape != cl.shape:
        raise ValueError("query_lens and context_lens differ in length")
    out = C.c_int32(0)
    check(load().pkv_prefill_partition_tokens(_i32p(ql), _i32p(cl), len(ql), num_q_heads, q_dtype,
                                              C.byref(out)))
    return out.value


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                 partition_tokens, algo, k_scale, v_scale, workspace, stream, allocate=True):
    torch = _torch()
    S, hq, d = q.shape
    nb, hkv, bs, _ = k_cache.shape
    d2 = _pool_head_dim(k_cache)
    if out.shape != q.shape or d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    need = pkv_decode_workspace_bytes(S, hq, d, max_context_len, partition_tokens)
    if need and workspace is None and allocate:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = C.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (_dev(out, "out"), _dtype_code(out), _dev(q, "q"), _dtype_code(q),
            _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(k_cache),
            _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
            _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
            _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, hq, hkv, d,
            bs, nb, float(scale), int(partition_tokens), int(algo), ws_ptr, ws_len,
            _stream(q, stream)), workspace


def pkv_paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens,
                               max_context_len: int, scale: float, partition_tokens: int = 0,
                               algo: int = PKV_ALGO_AUTO, k_scale=None, v_scale=None,
                               workspace=None, stream=None):
    """out, q: [S, Hq, D]; caches [NB, Hkv, BS, D] (int8 codes: int8; 4-bit
    codes: uint8 [NB, Hkv, BS, D / 2], both with float32 scales [NB, Hkv]);
    block_tables int32 [S, MB]; context_lens int32 [S].  Returns the
    workspace tensor used (or None)."""
    args, ws = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                            max_context_len, scale, partition_tokens, algo, k_scale, v_scale,
                            workspace, stream)
    check(load().pkv_paged_attention_decode(*args))
    return ws


def pkv_decode_step_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int,
                                    max_context_len: int, partition_tokens: int) -> int:
    return load().pkv_decode_step_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                  max_context_len, partition_tokens)


def pkv_paged_attention_decode_step(out, q, new_k, new_v, k_cache, v_cache, block_tables,
                                    context_lens, max_context_len: int, scale: float,
                                    partition_tokens: int = 0, algo: int = PKV_ALGO_AUTO,
                                    k_scale=None, v_scale=None, workspace=None, stream=None):
    """Append new_k / new_v [S, Hkv, D] (or None) at each sequence's last
    position and decode in the same launch; split rows are merged by the
    reduce kernel, or in the launch with PKV_MERGE_IN_KERNEL in algo (then
    the workspace, allocated zero-filled here when not given, must start
    with zero counters; calls leave them zero).  Returns the workspace."""
    torch = _torch()
    S, hq, d = q.shape
    nb, hkv, bs, _ = k_cache.shape
    if out.shape != q.shape or _pool_head_dim(k_cache) != d or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    if (new_k is None) != (new_v is None):
        raise ValueError("new_k and new_v are both given or both None")
    if new_k is not None:
        coded = k_cache.dtype in (torch.int8, torch.uint8)   # refused by the library
        for t in (new_k, new_v):
            if t.shape != (S, hkv, d) or (t.dtype != k_cache.dtype and not coded):
                raise ValueError("new rows must be [S, Hkv, D] in the pool's dtype")
    need = pkv_decode_step_workspace_bytes(S, hq, d, max_context_len, partition_tokens)
    if need and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(load().pkv_paged_attention_decode_step(
        _dev(out, "out"), _dtype_code(out), _dev(q, "q"), _dtype_code(q),
        _dev(new_k, "new_k"), _dev(new_v, "new_v"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dtype_code(k_cache), _dev(k_scale, "k_scale", torch.float32),
        _dev(v_scale, "v_scale", torch.float32), _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context_len), S, hq, hkv, d, bs, nb, float(scale), int(partition_tokens),
        int(algo), C.c_void_p(workspace.data_ptr()) if workspace is not None else None, ws_len,
        _stream(q, stream)))
    return workspace


def pkv_paged_attention_decode_partials(out, q, k_cache, v_cache, block_tables, context_lens,
                                        max_context_len: int, scale: float,
                                        partition_tokens: int = 0, algo: int = PKV_ALGO_AUTO,
                                        k_scale=None, v_scale=None, workspace=None, stream=None):
    args, ws = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                            max_context_len, scale, partition_tokens, algo, k_scale, v_scale,
                            workspace, stream)
    check(load().pkv_paged_attention_decode_partials(*args))
    return ws


def pkv_paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens,
                                       max_context_len: int, scale: float,
                                       partition_tokens: int = 0, algo: int = PKV_ALGO_AUTO,
                                       k_scale=None, v_scale=None, stream=None) -> None:
    """pkv_paged_attention_decode with the split-K partial results in the
    library's fixed per-GPU scratch (PKV_NOALLOC_SCRATCH_BYTES): no workspace
    argument and nothing allocated, here or in the library."""
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                           max_context_len, scale, partition_tokens, algo, k_scale, v_scale,
                           None, stream, allocate=False)
    check(load().pkv_paged_attention_decode_noalloc(*args[:-3], args[-1]))


def pkv_paged_attention_reduce(out, context_lens, max_context_len: int, partition_tokens: int,
                               workspace, stream=None) -> None:
    torch = _torch()
    S, hq, d = out.shape
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(load().pkv_paged_attention_reduce(
        _dev(out, "out"), _dtype_code(out), _dev(context_lens, "context_lens", torch.int32),
        int(max_context_len), S, hq, d, int(partition_tokens),
        C.c_void_p(workspace.data_ptr()) if workspace is not None else None, ws_len,
        _stream(out, stream)))


def pkv_prefill_workspace_bytes(num_query_tokens: int, num_q_heads: int, head_dim: int,
                                max_context_len: int, partition_tokens: int) -> int:
    return load().pkv_prefill_workspace_bytes(num_query_tokens, num_q_heads, head_dim,
                                              max_context_len, partition_tokens)


def pkv_paged_attention_prefill(out, q, k_cache, v_cache, block_tables, query_start_loc,
                                context_lens, max_query_len: int, max_context_len: int,
                                scale: float, k_scale=None, v_scale=None, stream=None,
                                partition_tokens: int = 0, workspace=None):
    """out, q: [Tq, Hq, D]; query_start_loc int32 [S+1]; context_lens int32 [S].
    Returns the workspace tensor used (or None)."""
    torch = _torch()
    Tq, hq, d = q.shape
    nb, hkv, bs, _ = k_cache.shape
    d2 = _pool_head_dim(k_cache)
    S = context_lens.shape[0]
    if out.shape != q.shape or d2 != d or query_start_loc.shape != (S + 1,):
        raise ValueError("shape mismatch")
    need = pkv_prefill_workspace_bytes(Tq, hq, d, int(max_context_len), int(partition_tokens))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = C.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(load().pkv_paged_attention_prefill(
        _dev(out, "out"), _dtype_code(out), _dev(q, "q"), _dtype_code(q), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dtype_code(k_cache), _dev(k_scale, "k_scale", torch.float32),
        _dev(v_scale, "v_scale", torch.float32), _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(query_start_loc, "query_start_loc", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), int(max_query_len), int(max_context_len),
        S, Tq, hq, hkv, d, bs, nb, float(scale), int(partition_tokens), ws_ptr, ws_len,
        _stream(q, stream)))
    return workspace


__all__ = sorted(set(__all__) | {n for n in dir() if n.startswith("pkv_")})
