"""Block manager model: free list, reference counts, sequences, copy-on-write.

What the pages fix:
  * a fixed pool of blocks; a free list initialised to all block ids, and
    allocation takes ids off its end (a stack), failing when it is empty
    ([cnnetsun] §2.1, the PagedKVCache sketch's allocate);
  * blocks are taken only when tokens arrive, so a sequence holds
    ceil(len / block_size) blocks and wastes less than one block
    ([kongchang] section "PagedAttention带来的性能收益");
  * several logical sequences may point at one physical block; a per-block
    reference count tracks them, and a sequence that must append into a block
    whose count exceeds 1 first gets a new block, copies the data and updates
    its table ([kongchang] section "KV Cache内存共享"; [aisoosoo] section
    "技术亮点"; [cnnetsun] §2.2);
  * blocks of a finished request return to the pool ([nxbn] §2.3).

Readings where the pages are silent (each one also holds in the C++ manager):
  * allocation is all-or-nothing: a request that cannot be met changes nothing;
  * ids of one allocation are returned in pop order, and a new sequence's
    blocks are its logical blocks 0..k-1 in that order;
  * freeing decrements the blocks of a sequence in logical order, and a block
    whose count reaches 0 is pushed back on the end of the free list;
  * a copy-on-write takes its destination before any new block of the same
    append; a full shared tail needs no copy (a fresh block is started);
  * in a batch of appends, sequences are handled in the order given, so of
    four beams sharing a partly filled tail the first three copy and the last
    writes in place;
  * sequence ids count up from 0 and are never reused.

Prefix caching: when several requests start with the same tokens (a system
prompt), their KV pages are reused instead of stored again
([cnnetsun] §2.2, the share_prefix sketch keyed by a hash of the prefix;
[aisoosoo] section "技术亮点": the scheduler hashes the prompt's tokens and
equal prefixes reuse KV pages without recomputation).  Readings:
  * the unit is a full block: block j of a sequence is found under the key
    (physical block of its logical block j - 1, or none for j = 0; the
    block_size token ids of block j), compared exactly (no false sharing);
  * seq_create_cached walks the prompt's full blocks and shares the longest
    run found from block 0 (each shared block's count + 1), then allocates
    the rest (all-or-nothing); it reports how many leading positions already
    hold their KV (block_size x shared blocks);
  * seq_publish registers a sequence's full blocks once the caller has
    written their KV; a key already present keeps its block (first writer
    wins), and a block is registered at most once;
  * an entry lives while its block is allocated: the cache holds no count of
    its own, and a block whose count reaches 0 leaves the cache;
  * lookup statistics count every full block of each cached create (looked
    up) and the ones shared (hits).
"""
from __future__ import annotations

import copy
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


class OutOfBlocks(Exception):
    pass


class Invalid(Exception):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int,
                 init_free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise Invalid("num_blocks and block_size must be positive")
        if init_free_order is None:
            self.free: List[int] = list(range(num_blocks))
        else:
            order = [int(b) for b in init_free_order]
            if sorted(order) != list(range(num_blocks)):
                raise Invalid("init_free_order must be a permutation of the block ids")
            self.free = order
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.rc = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.next_seq = 0
        self.cache: Dict[Tuple[int, Tuple[int, ...]], int] = {}
        self.cache_key: Dict[int, Tuple[int, Tuple[int, ...]]] = {}
        self.lookups = 0
        self.hits = 0

    # ---------------------------------------------------------------- blocks
    def alloc(self, k: int) -> List[int]:
        if k < 0:
            raise Invalid("negative count")
        if len(self.free) < k:
            raise OutOfBlocks(f"need {k} blocks, {len(self.free)} free")
        ids = []
        for _ in range(k):
            b = self.free.pop()
            self.rc[b] = 1
            ids.append(b)
        return ids

    def _check(self, b: int) -> None:
        if not (0 <= b < self.num_blocks) or self.rc[b] < 1:
            raise Invalid(f"block {b} is not allocated")

    def incref(self, b: int) -> None:
        self._check(b)
        self.rc[b] += 1

    def decref(self, b: int) -> None:
        self._check(b)
        self.rc[b] -= 1
        if self.rc[b] == 0:
            self.free.append(b)
            key = self.cache_key.pop(b, None)
            if key is not None:
                del self.cache[key]

    def num_free(self) -> int:
        return len(self.free)

    # ------------------------------------------------------------- sequences
    def _seq(self, sid: int) -> List[int]:
        if sid not in self.tables:
            raise Invalid(f"unknown sequence {sid}")
        return self.tables[sid]

    def seq_create(self, num_tokens: int) -> int:
        if num_tokens < 0:
            raise Invalid("negative length")
        nb = -(-num_tokens // self.block_size)
        blocks = self.alloc(nb)
        sid = self.next_seq
        self.next_seq += 1
        self.tables[sid] = blocks
        self.lens[sid] = num_tokens
        return sid

    def seq_create_cached(self, tokens: Sequence[int]) -> Tuple[int, int]:
        """New sequence over ``tokens``; returns (sequence id, positions whose
        KV is already in shared blocks)."""
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        shared: List[int] = []
        parent = -1
        for j in range(len(tokens) // bs):
            b = self.cache.get((parent, tuple(tokens[j * bs:(j + 1) * bs])))
            if b is None:
                break
            shared.append(b)
            parent = b
        need = -(-len(tokens) // bs) - len(shared)
        fresh = self.alloc(need)            # raises before any change
        for b in shared:
            self.rc[b] += 1
        sid = self.next_seq
        self.next_seq += 1
        self.tables[sid] = shared + fresh
        self.lens[sid] = len(tokens)
        self.lookups += len(tokens) // bs
        self.hits += len(shared)
        return sid, len(shared) * bs

    def seq_publish(self, sid: int, tokens: Sequence[int]) -> int:
        """Register the full blocks covered by ``tokens`` (the sequence's
        first len(tokens) positions); returns how many were newly
        registered."""
        table = self._seq(sid)
        tokens = [int(t) for t in tokens]
        if len(tokens) > self.lens[sid]:
            raise Invalid("more tokens than the sequence holds")
        bs = self.block_size
        added = 0
        for j in range(len(tokens) // bs):
            key = (table[j - 1] if j else -1, tuple(tokens[j * bs:(j + 1) * bs]))
            b = table[j]
            if key in self.cache or b in self.cache_key:
                continue
            self.cache[key] = b
            self.cache_key[b] = key
            added += 1
        return added

    def prefix_stats(self) -> dict:
        return {"cached_blocks": len(self.cache), "lookups": self.lookups, "hits": self.hits}

    def seq_fork(self, parent: int) -> int:
        table = self._seq(parent)
        for b in table:
            self.incref(b)
        sid = self.next_seq
        self.next_seq += 1
        self.tables[sid] = list(table)
        self.lens[sid] = self.lens[parent]
        return sid

    def _append_one(self, sid: int, cow: List[Tuple[int, int]]) -> int:
        table = self.tables[sid]
        n = self.lens[sid]
        bs = self.block_size
        if n % bs == 0:
            table.extend(self.alloc(1))
        elif self.rc[table[-1]] > 1:
            src = table[-1]
            dst = self.alloc(1)[0]
            cow.append((src, dst))
            self.decref(src)
            table[-1] = dst
        slot = table[n // bs] * bs + n % bs
        self.lens[sid] = n + 1
        return slot

    def _transaction(self, fn):
        saved = copy.deepcopy((self.free, self.rc, self.tables, self.lens))
        try:
            return fn()
        except OutOfBlocks:
            self.free, self.rc, self.tables, self.lens = saved
            raise

    def seq_append(self, sid: int, num_tokens: int = 1) -> Tuple[List[int], Optional[Tuple[int, int]]]:
        """Append ``num_tokens`` positions; returns their slots and the
        copy-on-write pair (src, dst) if one was needed, else None."""
        self._seq(sid)
        if num_tokens < 0:
            raise Invalid("negative count")

        def run():
            cow: List[Tuple[int, int]] = []
            slots = [self._append_one(sid, cow) for _ in range(num_tokens)]
            return slots, (cow[0] if cow else None)
        return self._transaction(run)

    def seq_append_batch(self, sids: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One new position per sequence, in the order given."""
        if len(set(sids)) != len(sids):
            raise Invalid("a sequence appears twice in one batch")
        for sid in sids:
            self._seq(sid)

        def run():
            cow: List[Tuple[int, int]] = []
            slots = [self._append_one(sid, cow) for sid in sids]
            return slots, cow
        return self._transaction(run)

    def seq_slots(self, sid: int, start: int, count: int) -> List[int]:
        table = self._seq(sid)
        n = self.lens[sid]
        if start < 0 or count < 0 or start + count > n:
            raise Invalid("positions out of range")
        bs = self.block_size
        return [table[p // bs] * bs + p % bs for p in range(start, start + count)]

    def seq_free(self, sid: int) -> None:
        table = self._seq(sid)
        for b in table:
            self.decref(b)
        del self.tables[sid]
        del self.lens[sid]

    def export(self, sids: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
        tables = np.full((len(sids), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(sids), dtype=np.int32)
        for i, sid in enumerate(sids):
            t = self._seq(sid)
            if len(t) > max_blocks:
                raise Invalid("max_blocks too small")
            tables[i, :len(t)] = t
            lens[i] = self.lens[sid]
        return tables, lens

    # ----------------------------------------------------------------- state
    def state(self) -> Tuple[List[int], List[int]]:
        return list(self.free), list(self.rc)

    def stats(self) -> dict:
        used = sum(1 for r in self.rc if r > 0)
        shared = sum(1 for r in self.rc if r > 1)
        logical = sum(len(t) for t in self.tables.values())
        waste = sum(len(t) * self.block_size - self.lens[s] for s, t in self.tables.items())
        return {"num_blocks": self.num_blocks, "free": len(self.free), "used": used,
                "shared": shared, "logical_blocks": logical, "waste_slots": waste,
                "num_seqs": len(self.tables)}


def adaptive_page_size(avg_seq_len: float) -> int:
    """Block size for a workload whose sequences average ``avg_seq_len``
    tokens: the rule [cnnetsun] §4.3 prints as an example (16 below 512
    tokens, 32 below 2048, 64 otherwise).  Reading for inputs the rule does
    not consider: NaN and negative averages get the smallest size."""
    if not avg_seq_len >= 512:
        return 16
    if avg_seq_len < 2048:
        return 32
    return 64
