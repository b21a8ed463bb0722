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
