"""Seeded synthetic workloads shaped like the pages' paged-KV serving cases.

Everything here is input preparation: random draws, rounding of fp32 draws
to the storage precision, the int8 storage encoding of the long-context case,
and laying values out in a block pool along a given placement.  The draw order
for every case is fixed: (1) context lengths, (2) pool permutation, (3) query
vectors, (4) K then V of each sequence in index order.

Storage conventions shared by both consumers:
  * float values are returned as float32 arrays holding exactly the stored
    value (bf16 / f16 values are rounded round-to-nearest-even first);
  * the pool is ``[num_blocks, kv_heads, block_size, head_dim]``;
  * slots that no token was written to hold NaN (int8: code 127 in allocated
    blocks, code -128 and a NaN scale in blocks no sequence owns), so any read
    of an unmasked slot shows up in the result;
  * 4-bit pools are random bytes ``[num_blocks, kv_heads, block_size,
    head_dim / 2]`` (every byte value, so every nibble) with scales drawn
    per owned (block, kv_head) and NaN for blocks no sequence owns.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16
UNUSED = np.float32(np.nan)
I8_UNUSED = np.int8(127)
I8_NEVER = np.int8(-128)

DTYPES = ("f32", "bf16", "f16")


# --------------------------------------------------------------------------
# rounding to storage precision
# --------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as float32.

    NaN stays NaN; finite inputs never overflow for the N(0,1) draws used here.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    # uint32 arithmetic: a finite pattern plus 0x8000 stays below 2^32; NaN
    # patterns may wrap and are restored below
    rounded = (bits >> np.uint32(16)) & np.uint32(1)
    rounded += bits
    rounded += np.uint32(0x7FFF)
    rounded &= np.uint32(0xFFFF0000)
    out = rounded.view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)
    raise ValueError(f"unknown float dtype {dtype!r}")


def storage_array(x: np.ndarray, dtype: str) -> np.ndarray:
    """The array whose bytes are the stored representation.

    f32 -> float32, f16 -> float16, bf16 -> uint16 (the high half of the
    float32 bit pattern; ``x`` must already be bf16-exact).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(dtype)


def from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# int8 storage encoding (per block and KV head, symmetric absmax / 127)
# --------------------------------------------------------------------------
def quantize_int8(x: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """Encode the filled rows of one (block, kv_head) tile.

    ``a = max|x|`` in fp32, ``s = a / 127`` (fp32 division), codes
    ``rint(x / s)`` (fp32 division, ties to even) clamped to [-127, 127];
    an all-zero tile gets ``s = 0`` and all-zero codes.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    s = np.float32(a / np.float32(127.0))
    if s == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    q = np.rint(x / s).astype(np.float32)
    return np.clip(q, -127, 127).astype(np.int8), s


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------
def draw_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform on [lo, hi] inclusive."""
    return rng.integers(lo, hi + 1, size=n).astype(np.int32)


def draw_permutation(rng: np.random.Generator, num_blocks: int) -> np.ndarray:
    return rng.permutation(num_blocks).astype(np.int32)


def draw_normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return round_to(rng.standard_normal(shape, dtype=np.float32), dtype)


def blocks_for(n: int, block_size: int = BLOCK_SIZE) -> int:
    return -(-int(n) // block_size)


def pool_size(lens: Sequence[int], factor: float = 1.25,
              block_size: int = BLOCK_SIZE) -> int:
    need = sum(blocks_for(n, block_size) for n in lens)
    return int(np.ceil(factor * need))


def place_by_permutation(lens: Sequence[int], perm: np.ndarray,
                         block_size: int = BLOCK_SIZE,
                         max_blocks: Optional[int] = None) -> np.ndarray:
    """Random physical placement: sequence s takes the next run of ``perm``.

    Returns int32 ``[S, max_blocks]`` padded with -1.
    """
    nbs = [blocks_for(n, block_size) for n in lens]
    mb = max_blocks if max_blocks is not None else max(1, max(nbs) if nbs else 1)
    tables = np.full((len(lens), mb), -1, dtype=np.int32)
    off = 0
    for s, nb in enumerate(nbs):
        if nb > mb:
            raise ValueError("max_blocks too small")
        tables[s, :nb] = perm[off:off + nb]
        off += nb
    if off > len(perm):
        raise ValueError("pool too small for the lengths")
    return tables


def scatter_rows(pool: np.ndarray, table_row: np.ndarray, rows: np.ndarray,
                 block_size: int, start: int = 0) -> None:
    """Lay logical rows ``[n, H, D]`` (positions start..start+n-1) into a pool
    image along one table row.  Input preparation for host-side pool images."""
    n = rows.shape[0]
    pos = np.arange(start, start + n)
    pool[table_row[pos // block_size], :, pos % block_size, :] = rows


@dataclass
class PagedCase:
    """One paged-attention input set (host arrays)."""
    dtype: str                      # storage dtype of q and float K/V
    q: np.ndarray                   # float32 [S or Tq, Hq, D]
    k_cache: np.ndarray             # float32 [NB, Hkv, BS, D] (NaN where unwritten)
    v_cache: np.ndarray
    block_tables: np.ndarray        # int32 [S, MB], -1 padded
    context_lens: np.ndarray        # int32 [S]
    scale: np.float32
    block_size: int = BLOCK_SIZE
    perm: Optional[np.ndarray] = None
    query_start_loc: Optional[np.ndarray] = None  # int32 [S+1] for prefill
    k_logical: Optional[List[np.ndarray]] = None  # per sequence [n, Hkv, D]
    v_logical: Optional[List[np.ndarray]] = None
    # int8 storage (present when kv is int8)
    k_i8: Optional[np.ndarray] = None
    v_i8: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None   # float32 [NB, Hkv]
    v_scale: Optional[np.ndarray] = None
    # 4-bit storage (present when kv is 4-bit): packed bytes and scales
    k_i4: Optional[np.ndarray] = None      # uint8 [NB, Hkv, BS, D / 2]
    v_i4: Optional[np.ndarray] = None
    k_scale4: Optional[np.ndarray] = None  # float32 [NB, Hkv]
    v_scale4: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return self.k_cache.shape[0]

    @property
    def kv_heads(self) -> int:
        return self.k_cache.shape[1]

    @property
    def head_dim(self) -> int:
        return self.k_cache.shape[3]


def draw_paged_kv(rng: np.random.Generator, tables: np.ndarray, lens, num_blocks: int,
                  kv_heads: int, head_dim: int, dtype: str, block_size: int = BLOCK_SIZE,
                  keep_logical: bool = False):
    """Draw K then V of each sequence (in index order) and lay them out."""
    k_cache = np.full((num_blocks, kv_heads, block_size, head_dim), UNUSED, np.float32)
    v_cache = np.full_like(k_cache, UNUSED)
    kl, vl = [], []
    for s, n in enumerate(lens):
        n = int(n)
        k = draw_normal(rng, (n, kv_heads, head_dim), dtype)
        v = draw_normal(rng, (n, kv_heads, head_dim), dtype)
        if n:
            scatter_rows(k_cache, tables[s], k, block_size)
            scatter_rows(v_cache, tables[s], v, block_size)
        if keep_logical:
            kl.append(k)
            vl.append(v)
    return k_cache, v_cache, (kl if keep_logical else None), (vl if keep_logical else None)


def int8_pool(cache: np.ndarray, tables: np.ndarray, lens,
              block_size: int = BLOCK_SIZE) -> Tuple[np.ndarray, np.ndarray]:
    """Int8 storage of a float pool: per (block, kv_head) codes and fp32 scales
    over the filled slots.  Unfilled slots of owned blocks hold code 127;
    blocks no sequence owns hold code -128 and a NaN scale."""
    nb, hkv, bs, d = cache.shape
    codes = np.full(cache.shape, I8_NEVER, np.int8)
    scales = np.full((nb, hkv), np.float32(np.nan), np.float32)
    filled = {}
    for s, n in enumerate(lens):
        n = int(n)
        for j in range(blocks_for(n, block_size)):
            b = int(tables[s, j])
            if b not in filled:
                filled[b] = min(block_size, n - j * block_size)
    if not filled:
        return codes, scales
    # every owned (block, kv head) tile at once: the same float32 steps as
    # quantize_int8, with rows past a block's filled count left out of the
    # maximum (held as 0) and stored as I8_UNUSED
    blk = np.fromiter(filled.keys(), np.int64, len(filled))
    nfill = np.fromiter(filled.values(), np.int64, len(filled))
    live = np.arange(bs)[None, :] < nfill[:, None]                       # [nblk, bs]
    for lo in range(0, len(blk), 4096):
        b, lv = blk[lo:lo + 4096], live[lo:lo + 4096]
        x = np.where(lv[:, None, :, None], cache[b], np.float32(0))         # [n, hkv, bs, d]
        a = np.abs(x).max(axis=(2, 3))                                       # [n, hkv]
        sc = (a / np.float32(127.0)).astype(np.float32)
        safe = np.where(sc == 0, np.float32(1), sc)
        q = np.clip(np.rint(x / safe[:, :, None, None]), -127, 127).astype(np.int8)
        q[sc == 0] = 0
        codes[b] = np.where(lv[:, None, :, None], q, I8_UNUSED)
        scales[b] = sc
    return codes, scales


def random_int4_pool(rng: np.random.Generator, tables: np.ndarray, lens, num_blocks: int,
                     kv_heads: int, head_dim: int, block_size: int = BLOCK_SIZE,
                     scale_range: Tuple[float, float] = (0.1, 0.3)):
    """A 4-bit pool as random bytes (uint8, every value) and float32 scales
    drawn U[scale_range] for the (block, kv_head) tiles some sequence owns,
    NaN elsewhere.  Draw order: bytes, then scales."""
    codes = rng.integers(0, 256, (num_blocks, kv_heads, block_size, head_dim // 2),
                         dtype=np.uint8)
    drawn = rng.uniform(scale_range[0], scale_range[1], (num_blocks, kv_heads)).astype(np.float32)
    scales = np.full((num_blocks, kv_heads), np.float32(np.nan), np.float32)
    for s, n in enumerate(lens):
        for j in range(blocks_for(int(n), block_size)):
            b = int(tables[s, j])
            scales[b] = drawn[b]
    return codes, scales


def decode_case(seed: int, num_seqs: int, q_heads: int, kv_heads: int, head_dim: int,
                lens: Optional[Sequence[int]] = None, len_range: Optional[Tuple[int, int]] = None,
                dtype: str = "bf16",
                block_size: int = BLOCK_SIZE, pool_factor: float = 1.25,
                num_blocks: Optional[int] = None, int8: bool = False,
                keep_logical: bool = False, max_blocks: Optional[int] = None,
                int4: bool = False) -> PagedCase:
    """Decode input: one query per sequence, K/V already cached.

    Either ``lens`` lists the context lengths (each includes the current
    token) or ``len_range=(lo, hi)`` draws them uniform on [lo, hi].  With
    ``int4`` a random 4-bit K pool then V pool are drawn after everything
    else (random_int4_pool).
    """
    rng = np.random.default_rng(seed)
    if len_range is not None:
        lens_arr = draw_lengths(rng, num_seqs, len_range[0], len_range[1])
    else:
        lens_arr = np.asarray(lens, dtype=np.int32)
        assert len(lens_arr) == num_seqs
    nb = num_blocks if num_blocks is not None else max(1, pool_size(lens_arr, pool_factor, block_size))
    perm = draw_permutation(rng, nb)
    tables = place_by_permutation(lens_arr, perm, block_size, max_blocks)
    q = draw_normal(rng, (num_seqs, q_heads, head_dim), dtype)
    k_cache, v_cache, kl, vl = draw_paged_kv(rng, tables, lens_arr, nb, kv_heads, head_dim,
                                             dtype, block_size, keep_logical)
    case = PagedCase(dtype=dtype, q=q, k_cache=k_cache, v_cache=v_cache, block_tables=tables,
                     context_lens=lens_arr, scale=np.float32(1.0 / np.sqrt(head_dim)),
                     block_size=block_size, perm=perm, k_logical=kl, v_logical=vl)
    if int8:
        case.k_i8, case.k_scale = int8_pool(k_cache, tables, lens_arr, block_size)
        case.v_i8, case.v_scale = int8_pool(v_cache, tables, lens_arr, block_size)
    if int4:
        case.k_i4, case.k_scale4 = random_int4_pool(rng, tables, lens_arr, nb, kv_heads, head_dim,
                                                    block_size)
        case.v_i4, case.v_scale4 = random_int4_pool(rng, tables, lens_arr, nb, kv_heads, head_dim,
                                                    block_size)
    return case


def prefill_case(seed: int, q_heads: int, kv_heads: int, head_dim: int,
                 chunks: Sequence[Tuple[int, int]], dtype: str = "bf16",
                 block_size: int = BLOCK_SIZE, pool_factor: float = 1.25,
                 keep_logical: bool = False) -> PagedCase:
    """Chunked-prefill input.  ``chunks`` lists (prior_cached, query_len) per
    sequence; the context of sequence s is prior + query_len and its K/V for
    every position (the chunk's own rows included) are in the pool."""
    rng = np.random.default_rng(seed)
    lens_arr = np.asarray([p + ql for p, ql in chunks], dtype=np.int32)
    qlens = np.asarray([ql for _, ql in chunks], dtype=np.int32)
    nb = max(1, pool_size(lens_arr, pool_factor, block_size))
    perm = draw_permutation(rng, nb)
    tables = place_by_permutation(lens_arr, perm, block_size)
    qsl = np.zeros(len(chunks) + 1, np.int32)
    qsl[1:] = np.cumsum(qlens)
    q = draw_normal(rng, (int(qsl[-1]), q_heads, head_dim), dtype)
    k_cache, v_cache, kl, vl = draw_paged_kv(rng, tables, lens_arr, nb, kv_heads, head_dim,
                                             dtype, block_size, keep_logical)
    return PagedCase(dtype=dtype, q=q, k_cache=k_cache, v_cache=v_cache, block_tables=tables,
                     context_lens=lens_arr, scale=np.float32(1.0 / np.sqrt(head_dim)),
                     block_size=block_size, perm=perm, query_start_loc=qsl,
                     k_logical=kl, v_logical=vl)


# --------------------------------------------------------------------------
# the five workload shapes
# --------------------------------------------------------------------------
TINY_LENS = (17, 50, 128, 200)


def tiny_decode(seed: int = 0, keep_logical: bool = True) -> PagedCase:
    """4 sequences, 8 MHA heads, head_dim 64, fp32, 64-block pool."""
    return decode_case(seed, 4, 8, 8, 64, lens=list(TINY_LENS), dtype="f32", num_blocks=64,
                       keep_logical=keep_logical)


def llama7b_decode(seed: int = 1, num_seqs: int = 64, lens=(128, 2048),
                   keep_logical: bool = False) -> PagedCase:
    """7B-shape decode: 32 MHA heads x 128, bf16, lengths U[128, 2048]."""
    return decode_case(seed, num_seqs, 32, 32, 128, len_range=lens, dtype="bf16",
                       keep_logical=keep_logical)


def gqa_long_decode(seed: int = 4, num_seqs: int = 16, lens=(8192, 32768), int8: bool = False,
                    keep_logical: bool = False, int4: bool = False) -> PagedCase:
    """Long-context GQA decode: 64 query heads over 8 KV heads, head_dim 128."""
    return decode_case(seed, num_seqs, 64, 8, 128, len_range=lens, dtype="bf16", int8=int8,
                       keep_logical=keep_logical, int4=int4)


@dataclass
class MixedStep:
    """Continuous-batching step: decode sequences plus prefill chunks.

    ``prior`` tokens of each sequence are already cached; ``new`` tokens
    (1 for decode, the chunk length for prefill) arrive this step and are
    written through the slot mapping before attention."""
    dtype: str
    prior: np.ndarray          # int32 [S]
    new: np.ndarray            # int32 [S]
    perm: np.ndarray           # free-list order of the pool
    num_blocks: int
    kv_heads: int
    head_dim: int
    q_heads: int
    prior_k: List[np.ndarray]  # per sequence [prior, Hkv, D]
    prior_v: List[np.ndarray]
    new_k: np.ndarray          # [T, Hkv, D], sequences in index order
    new_v: np.ndarray
    q: np.ndarray              # [T, Hq, D]
    scale: np.float32
    out_lens: Optional[np.ndarray] = None  # lognormal output lengths (long tail)


def mixed_step(seed: int = 2, num_decode: int = 48, decode_lens=(64, 4096),
               prefill_chunks=((0, 512), (512, 512), (1024, 512), (1536, 512)),
               q_heads: int = 32, kv_heads: int = 32, head_dim: int = 128,
               dtype: str = "bf16", pool_factor: float = 1.25) -> MixedStep:
    """48 decode sequences (context U[64, 4096]) and four 512-token chunks
    over 0/512/1024/1536 cached tokens.  Output lengths are lognormal
    (median 128, sigma 1, clipped to [1, 2048]) for multi-step use."""
    rng = np.random.default_rng(seed)
    dl = draw_lengths(rng, num_decode, decode_lens[0], decode_lens[1])
    prior = np.concatenate([dl - 1, np.asarray([p for p, _ in prefill_chunks], np.int32)])
    new = np.concatenate([np.ones(num_decode, np.int32),
                          np.asarray([c for _, c in prefill_chunks], np.int32)])
    total = prior + new
    nb = max(1, pool_size(total, pool_factor))
    perm = draw_permutation(rng, nb)
    T = int(new.sum())
    q = draw_normal(rng, (T, q_heads, head_dim), dtype)
    pk, pv = [], []
    new_k = np.empty((T, kv_heads, head_dim), np.float32)
    new_v = np.empty_like(new_k)
    off = 0
    for s in range(len(prior)):
        k = draw_normal(rng, (int(total[s]), kv_heads, head_dim), dtype)
        v = draw_normal(rng, (int(total[s]), kv_heads, head_dim), dtype)
        p = int(prior[s])
        pk.append(k[:p])
        pv.append(v[:p])
        new_k[off:off + int(new[s])] = k[p:]
        new_v[off:off + int(new[s])] = v[p:]
        off += int(new[s])
    out_lens = np.clip(np.rint(rng.lognormal(np.log(128.0), 1.0, size=len(prior))), 1, 2048)
    return MixedStep(dtype, prior.astype(np.int32), new, perm, nb, kv_heads, head_dim, q_heads,
                     pk, pv, new_k, new_v, q, np.float32(1.0 / np.sqrt(head_dim)),
                     out_lens.astype(np.int32))


@dataclass
class BeamCase:
    """Shared system prompt + per-request tokens, forked into beams."""
    dtype: str
    prefix_len: int
    request_lens: np.ndarray    # int32 [R] tokens after the shared prefix
    beam_width: int
    perm: np.ndarray
    num_blocks: int
    kv_heads: int
    q_heads: int
    head_dim: int
    prefix_k: np.ndarray        # [prefix_len, Hkv, D]
    prefix_v: np.ndarray
    req_k: List[np.ndarray]     # per request [n_r, Hkv, D]
    req_v: List[np.ndarray]
    beam_k: np.ndarray          # [R * beam_width, Hkv, D] the divergent token
    beam_v: np.ndarray
    q: np.ndarray               # [R * beam_width, Hq, D]
    scale: np.float32


def beam_cow(seed: int = 3, num_requests: int = 16, prefix_len: int = 1024,
             req_lens=(1, 200), beam_width: int = 4, q_heads: int = 32, kv_heads: int = 32,
             head_dim: int = 128, dtype: str = "bf16", pool_factor: float = 1.25) -> BeamCase:
    rng = np.random.default_rng(seed)
    rl = draw_lengths(rng, num_requests, req_lens[0], req_lens[1])
    # logical blocks if nothing were shared, plus one copy per beam tail
    logical = blocks_for(prefix_len) + sum(blocks_for(prefix_len + int(n)) for n in rl)
    nb = max(1, int(np.ceil(pool_factor * (logical + num_requests * beam_width))))
    perm = draw_permutation(rng, nb)
    nbeams = num_requests * beam_width
    q = draw_normal(rng, (nbeams, q_heads, head_dim), dtype)
    pk = draw_normal(rng, (prefix_len, kv_heads, head_dim), dtype)
    pv = draw_normal(rng, (prefix_len, kv_heads, head_dim), dtype)
    rk, rv = [], []
    for n in rl:
        rk.append(draw_normal(rng, (int(n), kv_heads, head_dim), dtype))
        rv.append(draw_normal(rng, (int(n), kv_heads, head_dim), dtype))
    bk = draw_normal(rng, (nbeams, kv_heads, head_dim), dtype)
    bv = draw_normal(rng, (nbeams, kv_heads, head_dim), dtype)
    return BeamCase(dtype, prefix_len, rl, beam_width, perm, nb, kv_heads, q_heads, head_dim,
                    pk, pv, rk, rv, bk, bv, q, np.float32(1.0 / np.sqrt(head_dim)))


def distinct_slots(rng: np.random.Generator, num_slots: int, count: int,
                   skip_fraction: float = 0.0) -> np.ndarray:
    """``count`` distinct slot indices below ``num_slots``; a fraction of them
    replaced by -1 (rows to skip)."""
    slots = rng.choice(num_slots, size=count, replace=False).astype(np.int32)
    if skip_fraction > 0:
        slots[rng.random(count) < skip_fraction] = -1
    return slots


# --------------------------------------------------------------------------
# prefix sharing: requests that start with (part of) one system prompt
# --------------------------------------------------------------------------
@dataclass
class PrefixCase:
    """Request r holds tokens ``prompts[r]``: the first ``shared_lens[r]``
    tokens of one system prompt, then tokens of its own.  K/V rows follow the
    tokens: a position whose token prefix equals the system prompt's holds the
    system prompt's row, every other position a fresh draw.  Own tokens of
    request r come from the id range [vocab * (r + 1), vocab * (r + 2)), so
    two requests' token sequences agree exactly on their common system-prompt
    part and differ right after it."""
    dtype: str
    perm: np.ndarray
    num_blocks: int
    kv_heads: int
    q_heads: int
    head_dim: int
    shared_lens: np.ndarray     # int32 [R]
    prompts: List[np.ndarray]   # int32 token ids, per request
    k: List[np.ndarray]         # per request [n_r, Hkv, D]
    v: List[np.ndarray]
    q: Optional[List[np.ndarray]]   # per request [n_r, Hq, D], or None
    next_k: np.ndarray          # [R, Hkv, D] one decode token per request
    next_v: np.ndarray
    next_q: np.ndarray          # [R, Hq, D]
    scale: np.float32


def prefix_sharing(seed: int = 6, num_requests: int = 32, system_len: int = 1024,
                   own_lens=(64, 256), shared_lens: Optional[Sequence[int]] = None,
                   q_heads: int = 32, kv_heads: int = 32, head_dim: int = 128,
                   dtype: str = "bf16", draw_q: bool = True, vocab: int = 32000,
                   pool_factor: float = 1.25) -> PrefixCase:
    """Draw order: own lengths, pool permutation, system tokens, system K then
    V, then per request its own tokens, K, V (and queries of every position),
    then the decode token's K, V and query of each request.  By default every
    request shares the whole system prompt."""
    rng = np.random.default_rng(seed)
    own = draw_lengths(rng, num_requests, own_lens[0], own_lens[1])
    sl = (np.full(num_requests, system_len, np.int32) if shared_lens is None
          else np.asarray(shared_lens, np.int32))
    assert len(sl) == num_requests and sl.max() <= system_len and own.min() >= 1
    nb = max(1, int(np.ceil(pool_factor * sum(blocks_for(int(a + b) + 1)
                                             for a, b in zip(sl, own)))))
    perm = draw_permutation(rng, nb)
    sys_tok = rng.integers(0, vocab, system_len).astype(np.int32)
    sys_k = draw_normal(rng, (system_len, kv_heads, head_dim), dtype)
    sys_v = draw_normal(rng, (system_len, kv_heads, head_dim), dtype)
    prompts, ks, vs, qs = [], [], [], []
    for r in range(num_requests):
        m, n = int(sl[r]), int(own[r])
        t = rng.integers(vocab * (r + 1), vocab * (r + 2), n).astype(np.int32)
        k = draw_normal(rng, (n, kv_heads, head_dim), dtype)
        v = draw_normal(rng, (n, kv_heads, head_dim), dtype)
        prompts.append(np.concatenate([sys_tok[:m], t]))
        ks.append(np.concatenate([sys_k[:m], k]))
        vs.append(np.concatenate([sys_v[:m], v]))
        if draw_q:
            qs.append(draw_normal(rng, (m + n, q_heads, head_dim), dtype))
    nk = draw_normal(rng, (num_requests, kv_heads, head_dim), dtype)
    nv = draw_normal(rng, (num_requests, kv_heads, head_dim), dtype)
    nq = draw_normal(rng, (num_requests, q_heads, head_dim), dtype)
    return PrefixCase(dtype, perm, nb, kv_heads, q_heads, head_dim, sl, prompts, ks, vs,
                      qs if draw_q else None, nk, nv, nq, np.float32(1.0 / np.sqrt(head_dim)))
