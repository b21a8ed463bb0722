"""Int8 and 4-bit storage of KV blocks, as its definition — TEST
INFRASTRUCTURE ONLY.

The cnnetsun.cn page ("别再让GPU内存拖后腿了…") lists INT8 KV in its memory
compression table (§3.2 内存压缩技术: a quarter of fp32's bytes) and 4-bit
KV beside it (an eighth of fp32's bytes, 87.5% less); for long documents it
turns INT8 on for the historical pages (§4.3 典型场景优化策略).  The encoding
itself is not on the pages.  Reading taken here: symmetric codes per
(block, KV head), over the block's filled rows, with Q = 127 for int8 and
Q = 7 for 4-bit,

    a     = max |x|                          (float32)
    s     = float32(a / Q)                   (IEEE division, nearest even)
    code  = 0                                   if s == 0
          = clip(rint(float32(x / s)), -Q, Q)   otherwise
                                             (IEEE division; rint ties to even)

and rows past the filled count get code 0.  A scale below the smallest
normal float32 (a block whose values are all below about 1.5e-36 times Q)
counts as zero: such a block stores all-zero codes.

4-bit codes are stored two to a byte: element 2i of a row in the low
nibble of byte i and element 2i + 1 in the high nibble, each as a 4-bit
two's complement value (-8 is never written).

Everything is float32 arithmetic, as the definition states: the result is
unique bit for bit.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

SMALLEST_NORMAL = np.float32(np.finfo(np.float32).tiny)
INT8_MAX = 127   # largest int8 code
INT4_MAX = 7     # largest 4-bit code


def quantize_tile(x: np.ndarray, filled: int, qmax: int = INT8_MAX) -> Tuple[np.ndarray, np.float32]:
    """Codes ``int8 [rows, D]`` in [-qmax, qmax] and the scale of one
    (block, KV head) tile whose first ``filled`` rows hold data."""
    x = np.asarray(x, dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.int8)
    filled = int(filled)
    if filled <= 0:
        return codes, np.float32(0)
    rows = x[:filled]
    a = np.float32(np.max(np.abs(rows)))
    s = np.float32(a / np.float32(qmax))
    if s < SMALLEST_NORMAL:
        return codes, np.float32(0)
    q = np.rint((rows / s).astype(np.float32))
    codes[:filled] = np.clip(q, -qmax, qmax).astype(np.int8)
    return codes, s


def quantize_blocks(pool: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                    blocks: Sequence[int], filled: Sequence[int], qmax: int = INT8_MAX):
    """Encode the listed blocks of a float pool ``[NB, H, BS, D]`` (values
    exactly as stored) into copies of an int8 pool and its ``[NB, H]``
    scales; blocks not listed keep what they held.  A filled count of 0
    leaves the block untouched."""
    out_codes = np.array(codes, dtype=np.int8, copy=True)
    out_scales = np.array(scales, dtype=np.float32, copy=True)
    for b, f in zip(blocks, filled):
        b, f = int(b), int(f)
        if f <= 0:
            continue
        for h in range(pool.shape[1]):
            out_codes[b, h], out_scales[b, h] = quantize_tile(pool[b, h], f, qmax)
    return out_codes, out_scales


def runs_of(slots: Sequence[int], block_size: int):
    """Split a slot mapping into runs: maximal stretches of consecutive
    tokens whose slots are consecutive rows of one block.  Yields (first
    token, block, first row, number of rows); slots < 0 are skipped."""
    t, n = 0, len(slots)
    while t < n:
        s = int(slots[t])
        if s < 0:
            t += 1
            continue
        b, r = s // block_size, s % block_size
        k = 1
        while (t + k < n and int(slots[t + k]) >= 0 and int(slots[t + k]) // block_size == b
               and int(slots[t + k]) == s + k):
            k += 1
        yield t, b, r, k
        t += k


def append_tile(codes: np.ndarray, scale: np.float32, row0: int, new_rows: np.ndarray,
                qmax: int = INT8_MAX):
    """Quantise-on-write of one (block, KV head) tile: rows [0, row0) hold
    codes under ``scale`` and ``new_rows`` (float32, exactly as stored) go to
    rows row0, row0 + 1, ....  Returns the tile's new codes and scale.

    Reading (the pages name INT8 KV but no encoding, cnnetsun.cn §3.2 and
    §4.3): the scale only grows.  s_new = max(s_old, float32(a / qmax)) with
    a = max |new rows| (s_old counts as 0 when row0 == 0); a scale below the
    smallest normal float32 counts as 0.  When the scale grows, each existing
    code c is re-encoded from its value: rint(float32(float32(c * s_old) /
    s_new)), clamped to [-qmax, qmax]; new rows encode as rint(float32(x /
    s_new)), clamped.  With row0 == 0 this is quantize_tile over the new
    rows."""
    codes = np.array(codes, dtype=np.int8, copy=True)
    new_rows = np.asarray(new_rows, dtype=np.float32)
    k = new_rows.shape[0]
    s_old = np.float32(scale) if row0 > 0 else np.float32(0)
    a = np.float32(np.max(np.abs(new_rows))) if k else np.float32(0)
    s_new = max(s_old, np.float32(a / np.float32(qmax)))
    if s_new < SMALLEST_NORMAL:
        s_new = np.float32(0)
    if s_new == 0:
        codes[row0:row0 + k] = 0
        return codes, np.float32(s_new if row0 == 0 else s_old)
    if s_new > s_old and row0 > 0:
        old = codes[:row0].astype(np.float32)
        vals = (old * s_old).astype(np.float32)
        codes[:row0] = np.clip(np.rint((vals / s_new).astype(np.float32)), -qmax, qmax).astype(np.int8)
    q = np.rint((new_rows / s_new).astype(np.float32))
    codes[row0:row0 + k] = np.clip(q, -qmax, qmax).astype(np.int8)
    return codes, np.float32(s_new)


def reshape_and_cache_int8(key: np.ndarray, value: np.ndarray, k_codes: np.ndarray,
                           v_codes: np.ndarray, k_scale: np.ndarray, v_scale: np.ndarray,
                           slots: Sequence[int], block_size: int, qmax: int = INT8_MAX):
    """Write new tokens' K/V ``[T, H, D]`` (float32, exactly as stored) into
    int8 pools ``[NB, H, BS, D]`` with per-(block, head) scales ``[NB, H]``,
    run by run (see runs_of): each run's block takes its rows below the
    run's first row as already written and encodes the run with
    append_tile.  Returns new copies of the four arrays."""
    kc, vc = np.array(k_codes, copy=True), np.array(v_codes, copy=True)
    ks, vs = np.array(k_scale, np.float32, copy=True), np.array(v_scale, np.float32, copy=True)
    for t0, b, r0, k in runs_of(slots, block_size):
        for h in range(kc.shape[1]):
            kc[b, h], ks[b, h] = append_tile(kc[b, h], ks[b, h], r0, key[t0:t0 + k, h], qmax)
            vc[b, h], vs[b, h] = append_tile(vc[b, h], vs[b, h], r0, value[t0:t0 + k, h], qmax)
    return kc, vc, ks, vs


# ------------------------------------------------------------------ 4-bit
def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Codes in [-8, 7], last axis even, to bytes: element 2i in the low
    nibble of byte i, element 2i + 1 in the high nibble (two's complement)."""
    c = np.asarray(codes).astype(np.int64)
    if c.shape[-1] % 2:
        raise ValueError("4-bit rows need an even length")
    if c.size and (c.min() < -8 or c.max() > 7):
        raise ValueError("4-bit codes lie in [-8, 7]")
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: bytes [..., D/2] to int8 codes [..., D]."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    lo, hi = b & 0xF, b >> 4
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int64)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out.astype(np.int8)


def quantize_blocks_int4(pool: np.ndarray, packed: np.ndarray, scales: np.ndarray,
                         blocks: Sequence[int], filled: Sequence[int]):
    """quantize_blocks with 4-bit codes: ``packed`` is the uint8 pool
    ``[NB, H, BS, D/2]``; returns new packed codes and scales."""
    codes, sc = quantize_blocks(pool, unpack_int4(packed), scales, blocks, filled, INT4_MAX)
    return pack_int4(codes), sc


def reshape_and_cache_int4(key: np.ndarray, value: np.ndarray, k_packed: np.ndarray,
                           v_packed: np.ndarray, k_scale: np.ndarray, v_scale: np.ndarray,
                           slots: Sequence[int], block_size: int):
    """reshape_and_cache_int8 into packed 4-bit pools ``[NB, H, BS, D/2]``."""
    kc, vc, ks, vs = reshape_and_cache_int8(key, value, unpack_int4(k_packed), unpack_int4(v_packed),
                                            k_scale, v_scale, slots, block_size, INT4_MAX)
    return pack_int4(kc), pack_int4(vc), ks, vs


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bits: int) -> float:
    """Bytes one token's K and V take over all layers with ``bits``-bit
    elements (scales not counted): 2 x layers x kv_heads x head_dim x bits / 8
    (kongchang.com, 自回归生成的内存开销, with the element width of the
    cnnetsun.cn compression table, §3.2)."""
    return 2 * layers * kv_heads * head_dim * bits / 8
