"""Paged attention, written as its plain definition in float64.

A sequence's keys and values live in fixed-size blocks scattered through a
global pool; the block table maps logical block j of sequence s to a physical
block id ([kongchang] section "PagedAttention的核心创新"; [cnnetsun] §2.1;
[nxbn] §2.2).  Attention over such a cache is ordinary softmax attention over
the logical sequence: for each table entry compute the query's scores against
that page, concatenate, apply softmax to the scores divided by sqrt(dim), and
sum the pages' value rows with those weights ([cnnetsun] §3.1).

The oracle therefore (1) gathers the cache through the table into contiguous
K/V of the logical sequence, widened exactly to float64, and (2) runs the
textbook computation on them.  Readings of points the pages leave open:
  * only the first ``context_len`` positions count (the unfilled tail of the
    last block is not part of the sequence);
  * the scale is an explicit fp32 argument (1/sqrt(head_dim) in every
    workload), widened exactly to float64;
  * in decode, ``context_len`` already includes the current token: its K/V is
    appended to the cache before attention ([nxbn] section 一);
  * grouped heads are contiguous: query head h reads KV head h // (Hq / Hkv);
  * int8 storage decodes as code * scale[block][kv_head];
  * a sequence with context 0 has an all-zero output row.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def gather(cache: np.ndarray, table_row: np.ndarray, n: int, block_size: int,
           scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Contiguous ``[n, H, D]`` float64 K (or V) of one logical sequence.

    Position p lives in physical block ``table_row[p // block_size]`` at row
    ``p % block_size`` ([cnnetsun] §2.1; [nxbn] §2.2).  With int8 storage the
    row decodes as ``float64(code) * float64(scale[block][head])``.
    """
    pos = np.arange(int(n))
    blocks = np.asarray(table_row)[pos // block_size]
    if blocks.size and (blocks.min() < 0 or blocks.max() >= cache.shape[0]):
        raise ValueError("a table entry inside the context names no block of the pool")
    rows = np.asarray(cache)[blocks, :, pos % block_size, :].astype(np.float64)
    if scale is not None:
        rows = rows * np.asarray(scale, dtype=np.float64)[blocks][:, :, None]
    return rows


def softmax_weights(x: np.ndarray) -> np.ndarray:
    """Softmax of a score vector: exp(x - max x) / sum(exp(x - max x)).

    Subtracting the maximum leaves the definition's value unchanged and keeps
    exp finite ([cnnetsun] §3.1 applies softmax over the concatenated scores).
    """
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - np.max(x))
    return e / np.sum(e)


def attend(qvec: np.ndarray, K: np.ndarray, V: np.ndarray, scale) -> np.ndarray:
    """One query row against contiguous keys/values ``[n, D]`` (float64)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    x = np.float64(scale) * (K @ np.asarray(qvec, dtype=np.float64))
    return softmax_weights(x) @ V


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray, scale,
           block_size: int = 16, k_scale: Optional[np.ndarray] = None,
           v_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Decode attention: one query per sequence at position ``n - 1`` over keys
    ``[0, n)``, ``n = context_lens[s]``.  Returns float64 ``[S, Hq, D]``."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        n = int(context_lens[s])
        K = gather(k_cache, block_tables[s], n, block_size, k_scale)
        V = gather(v_cache, block_tables[s], n, block_size, v_scale)
        for h in range(Hq):
            g = h // G
            out[s, h] = attend(q[s, h], K[:, g, :], V[:, g, :], scale)
    return out


def decode_weights(q: np.ndarray, k_cache: np.ndarray, block_tables: np.ndarray,
                   context_lens: np.ndarray, scale, s: int, h: int,
                   block_size: int = 16, k_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """The softmax weights of (sequence s, query head h) in decode."""
    Hq = q.shape[1]
    G = Hq // k_cache.shape[1]
    n = int(context_lens[s])
    K = gather(k_cache, block_tables[s], n, block_size, k_scale)[:, h // G, :]
    return softmax_weights(np.float64(scale) * (K @ q[s, h].astype(np.float64)))


def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
            block_tables: np.ndarray, query_start_loc: np.ndarray,
            context_lens: np.ndarray, scale, block_size: int = 16,
            k_scale: Optional[np.ndarray] = None,
            v_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Chunked prefill: the query rows of sequence s are its last ``qlen``
    positions.  Row i sits at position ``P_i = n - qlen + i`` and attends keys
    ``[0, P_i]`` (causal over absolute positions; the chunk's own K/V are in
    the cache).  Prefill and decode steps share one batch ([nxbn] §3.2;
    [cnnetsun] §4.1 enables chunking of long prompts).

    ``q`` is ``[Tq, Hq, D]`` with the rows of sequence s at
    ``query_start_loc[s] : query_start_loc[s+1]``.  Returns float64.
    """
    Tq, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    S = len(context_lens)
    for s in range(S):
        a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
        qlen = b - a
        n = int(context_lens[s])
        if qlen == 0:
            continue
        if qlen > n:
            raise ValueError("a chunk cannot be longer than its context")
        K = gather(k_cache, block_tables[s], n, block_size, k_scale)
        V = gather(v_cache, block_tables[s], n, block_size, v_scale)
        for i in range(qlen):
            P = n - qlen + i
            for h in range(Hq):
                g = h // G
                out[a + i, h] = attend(q[a + i, h], K[:P + 1, g, :], V[:P + 1, g, :], scale)
    return out
