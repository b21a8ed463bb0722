"""Pins of the block-manager model.

* the pages' printed allocator behaviour (golden fixture, worked by hand from
  the cnnetsun.cn sketch);
* invariants that a brute-force recount checks after every operation of
  random operation sequences: each block's reference count equals the number
  of live block tables holding it, free and used blocks partition the pool,
  a sequence holds exactly ceil(len / block_size) blocks (waste below one
  block), and an append never writes into a block someone else still holds;
* the copy-on-write rules on concrete beam cases.
"""
import json
import os
import random

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.allocator import BlockManagerModel, Invalid, OutOfBlocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pages_lifo_allocation_golden():
    g = json.load(open(os.path.join(GOLDEN, "allocator_lifo.json")))
    bm = BlockManagerModel(g["num_blocks"], 16)
    for step in g["steps"]:
        if "error" in step:
            with pytest.raises(OutOfBlocks):
                bm.alloc(step["n"])
        else:
            assert bm.alloc(step["n"]) == step["ids"]
        assert bm.state()[0] == step["free_after"]


def check_invariants(bm: BlockManagerModel):
    free, rc = bm.state()
    assert len(set(free)) == len(free)
    holders = [0] * bm.num_blocks
    for sid, table in bm.tables.items():
        assert len(set(table)) == len(table)
        assert len(table) == -(-bm.lens[sid] // bm.block_size)
        waste = len(table) * bm.block_size - bm.lens[sid]
        assert 0 <= waste <= bm.block_size - 1
        for b in table:
            holders[b] += 1
    assert holders == rc
    assert set(free) == {b for b in range(bm.num_blocks) if rc[b] == 0}
    assert len(free) + sum(1 for r in rc if r > 0) == bm.num_blocks


def slot_block(bm, slot):
    return slot // bm.block_size


ops = st.lists(st.tuples(st.sampled_from(["create", "fork", "append", "append_n", "batch", "free"]),
                         st.integers(0, 1 << 30), st.integers(0, 40)), min_size=1, max_size=60)


@settings(max_examples=150, deadline=None)
@given(ops, st.integers(1, 48), st.sampled_from([1, 4, 16]), st.integers(0, 1 << 30))
def test_random_operation_sequences_keep_invariants(seq, nblocks, bs, seed):
    perm = list(np.random.default_rng(seed).permutation(nblocks))
    bm = BlockManagerModel(nblocks, bs, perm)
    live = []
    for op, pick, n in seq:
        before = (bm.state(), {k: list(v) for k, v in bm.tables.items()}, dict(bm.lens))
        try:
            if op == "create":
                live.append(bm.seq_create(n))
            elif op == "fork" and live:
                live.append(bm.seq_fork(live[pick % len(live)]))
            elif op in ("append", "append_n") and live:
                sid = live[pick % len(live)]
                parent_tables = {k: list(v) for k, v in bm.tables.items() if k != sid}
                slots, cow = bm.seq_append(sid, 1 if op == "append" else n % 5)
                for sl in slots:
                    assert bm.rc[slot_block(bm, sl)] == 1  # never write into a shared block
                    assert slot_block(bm, sl) in bm.tables[sid]
                for k, v in parent_tables.items():
                    assert bm.tables[k] == v       # nobody else's table changes
                if cow is not None:
                    assert bm.tables[sid][-1] == cow[1] or cow[1] in bm.tables[sid]
            elif op == "batch" and live:
                k = 1 + pick % len(live)
                sids = random.Random(pick).sample(live, k)
                slots, cows = bm.seq_append_batch(sids)
                assert len(set(slots)) == len(slots)
                for sl in slots:
                    assert bm.rc[slot_block(bm, sl)] == 1
                dsts = [d for _, d in cows]
                assert len(set(dsts)) == len(dsts)
                assert not set(dsts) & {s_ for s_, _ in cows}
            elif op == "free" and live:
                sid = live.pop(pick % len(live))
                bm.seq_free(sid)
        except OutOfBlocks:
            after = (bm.state(), {k: list(v) for k, v in bm.tables.items()}, dict(bm.lens))
            assert after == before  # all-or-nothing
        check_invariants(bm)
    for sid in live:
        bm.seq_free(sid)
    check_invariants(bm)
    assert bm.num_free() == nblocks


def test_slots_address_the_position_in_the_table():
    bm = BlockManagerModel(40, 16, list(np.random.default_rng(1).permutation(40)))
    sid = bm.seq_create(37)
    table = bm.tables[sid]
    slots = bm.seq_slots(sid, 0, 37)
    for p, sl in enumerate(slots):
        assert sl // 16 == table[p // 16] and sl % 16 == p % 16
    new, cow = bm.seq_append(sid, 30)
    assert cow is None
    for i, sl in enumerate(new):
        p = 37 + i
        assert sl // 16 == bm.tables[sid][p // 16] and sl % 16 == p % 16


def test_pool_exhaustion_at_exact_capacity():
    bm = BlockManagerModel(64, 16)
    with pytest.raises(OutOfBlocks):
        bm.seq_create(16 * 64 + 1)
    root = bm.seq_create(16 * 64)
    assert bm.num_free() == 0 and len(bm.tables[root]) == 64
    with pytest.raises(OutOfBlocks):
        bm.seq_append(root, 1)


def test_copy_on_write_order_for_four_beams():
    bm = BlockManagerModel(32, 16)
    req = bm.seq_create(21)                 # 2 blocks, tail holds 5 tokens
    beams = [req] + [bm.seq_fork(req) for _ in range(3)]
    tail = bm.tables[req][-1]
    assert bm.rc[tail] == 4
    slots, cows = bm.seq_append_batch(beams)
    assert [c[0] for c in cows] == [tail, tail, tail]
    assert bm.tables[beams[3]][-1] == tail      # last beam writes in place
    assert bm.rc[tail] == 1
    for b, sl in zip(beams, slots):
        assert sl == bm.tables[b][-1] * 16 + 5
    check_invariants(bm)


def test_full_shared_tail_needs_no_copy():
    bm = BlockManagerModel(16, 16)
    a = bm.seq_create(32)
    b = bm.seq_fork(a)
    slots, cow = bm.seq_append(b, 1)
    assert cow is None and bm.lens[b] == 33
    assert bm.tables[b][:2] == bm.tables[a]
    check_invariants(bm)


def test_out_of_blocks_changes_nothing():
    bm = BlockManagerModel(5, 4)
    a = bm.seq_create(7)                     # 2 blocks
    b = bm.seq_fork(a)
    before = (bm.state(), {k: list(v) for k, v in bm.tables.items()}, dict(bm.lens))
    with pytest.raises(OutOfBlocks):
        bm.seq_append(a, 20)                 # needs CoW + 5 new blocks > 3 free
    assert (bm.state(), {k: list(v) for k, v in bm.tables.items()}, dict(bm.lens)) == before
    with pytest.raises(OutOfBlocks):
        bm.seq_create(13)
    assert (bm.state(), {k: list(v) for k, v in bm.tables.items()}, dict(bm.lens)) == before


def test_invalid_operations_are_rejected():
    bm = BlockManagerModel(4, 16)
    with pytest.raises(Invalid):
        bm.decref(0)
    with pytest.raises(Invalid):
        bm.incref(9)
    with pytest.raises(Invalid):
        bm.seq_fork(3)
    a = bm.seq_create(3)
    with pytest.raises(Invalid):
        bm.seq_append_batch([a, a])
    with pytest.raises(Invalid):
        BlockManagerModel(4, 16, [0, 1, 1, 2])


def test_free_returns_blocks_in_logical_order():
    bm = BlockManagerModel(8, 2)
    a = bm.seq_create(6)                     # takes 7, 6, 5
    assert bm.tables[a] == [7, 6, 5]
    bm.seq_free(a)
    assert bm.state()[0] == [0, 1, 2, 3, 4, 7, 6, 5]
    assert bm.alloc(2) == [5, 6]


# ------------------------------------------------------------ prefix caching
def test_prefix_cache_golden():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "prefix_cache.json")))
    m = BlockManagerModel(g["num_blocks"], g["block_size"])
    ids = {}
    for st in g["steps"]:
        if st["op"] == "create_cached":
            sid, cached = m.seq_create_cached(st["tokens"])
            ids[st["name"]] = sid
            assert m.tables[sid] == st["table"] and cached == st["cached"], st
        elif st["op"] == "publish":
            assert m.seq_publish(ids[st["name"]], st["tokens"]) == st["added"]
        elif st["op"] == "free":
            m.seq_free(ids[st["name"]])
            assert m.free == st["free_after"], st
        else:
            ps = m.prefix_stats()
            assert (ps["lookups"], ps["hits"], ps["cached_blocks"]) == (
                st["lookups"], st["hits"], st["cached_blocks"])


@pytest.mark.parametrize("seed", range(6))
def test_prefix_cache_never_shares_different_prefixes(seed):
    """Random creates from a few prompt families, publishes, forks, appends
    and frees.  Whenever two live sequences hold the same physical block at
    logical index j, they agree on every token up to the end of block j;
    cache entries name live blocks only; counts recount by brute force."""
    rng = np.random.default_rng(seed)
    bs = 4
    m = BlockManagerModel(64, bs, list(rng.permutation(64)))
    toks = {}
    families = [list(rng.integers(0, 5, 24)) for _ in range(3)]
    for _ in range(200):
        op = rng.integers(0, 5)
        try:
            if op <= 1 or not m.tables:
                f = families[rng.integers(0, 3)]
                n = int(rng.integers(1, 24))
                tail = list(rng.integers(0, 5, int(rng.integers(0, 6))))
                t = f[:n] + tail
                sid, cached = m.seq_create_cached(t)
                assert cached % bs == 0 and cached <= len(t)
                toks[sid] = t
            elif op == 2:
                sid = int(rng.choice(list(m.tables)))
                m.seq_publish(sid, toks[sid][:int(rng.integers(0, len(toks[sid]) + 1))])
            elif op == 3:
                sid = int(rng.choice(list(m.tables)))
                new = [int(x) for x in rng.integers(0, 5, int(rng.integers(1, 4)))]
                m.seq_append(sid, len(new))
                toks[sid] = toks[sid] + new
            else:
                sid = int(rng.choice(list(m.tables)))
                m.seq_free(sid)
                del toks[sid]
        except OutOfBlocks:
            pass
        # invariants
        for b, key in m.cache_key.items():
            assert m.rc[b] > 0 and m.cache[key] == b
        count = [0] * 64
        for t in m.tables.values():
            for b in t:
                count[b] += 1
        assert count == m.rc
        live = list(m.tables)
        for i in live:
            for k in live:
                if i >= k:
                    continue
                ti, tk = m.tables[i], m.tables[k]
                for j in range(min(len(ti), len(tk))):
                    if ti[j] == tk[j]:
                        end = min((j + 1) * bs, m.lens[i], m.lens[k])
                        assert toks[i][:end] == toks[k][:end], (i, k, j)


# ------------------------------------------------------------ adaptive block size
def test_adaptive_page_size_golden():
    import json
    import os
    from oracle.allocator import adaptive_page_size
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "adaptive_block_size.json")))
    for avg, want in g["cases"]:
        assert adaptive_page_size(avg) == want, avg


def test_adaptive_page_size_is_monotone_and_in_the_pages_range():
    from oracle.allocator import adaptive_page_size
    xs = np.sort(np.random.default_rng(0).uniform(0, 1e5, 2000))
    sizes = [adaptive_page_size(x) for x in xs]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    assert set(sizes) == {16, 32, 64}
    assert adaptive_page_size(float("nan")) == 16 and adaptive_page_size(-5) == 16
