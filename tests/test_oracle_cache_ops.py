"""Pins of the cache-write and block-copy oracle, and the copy-on-write
invariant at the attention level (a parent's output does not change when its
children fork, copy the shared tail and append)."""
import numpy as np

from oracle import attention as A
from oracle import cache_ops as C
from oracle.allocator import BlockManagerModel
from synth import workloads as W


def _pool(nb=12, h=3, bs=16, d=8):
    return (np.full((nb, h, bs, d), np.nan, np.float32),
            np.full((nb, h, bs, d), np.nan, np.float32))


def test_reshape_and_cache_round_trip_and_untouched_slots():
    rng = np.random.default_rng(0)
    kc, vc = _pool()
    kc[:] = rng.standard_normal(kc.shape).astype(np.float32)
    slots = W.distinct_slots(rng, 12 * 16, 40, skip_fraction=0.2)
    key = rng.standard_normal((40, 3, 8)).astype(np.float32)
    val = rng.standard_normal((40, 3, 8)).astype(np.float32)
    k2, v2 = C.reshape_and_cache(key, val, kc, vc, slots, 16)
    flat_k = k2.transpose(0, 2, 1, 3).reshape(-1, 3, 8)   # [slot, H, D]
    flat_v = v2.transpose(0, 2, 1, 3).reshape(-1, 3, 8)
    for t, sl in enumerate(slots):
        if sl >= 0:
            assert np.array_equal(flat_k[sl], key[t]) and np.array_equal(flat_v[sl], val[t])
    written = set(int(s) for s in slots if s >= 0)
    other = [s for s in range(12 * 16) if s not in written]
    old_k = kc.transpose(0, 2, 1, 3).reshape(-1, 3, 8)
    old_v = vc.transpose(0, 2, 1, 3).reshape(-1, 3, 8)
    assert np.array_equal(flat_k[other].view(np.uint32), old_k[other].view(np.uint32))
    assert np.array_equal(flat_v[other].view(np.uint32), old_v[other].view(np.uint32))


def test_copy_blocks_copies_pairs_and_nothing_else():
    rng = np.random.default_rng(1)
    kc = rng.standard_normal((10, 2, 16, 4)).astype(np.float32)
    vc = rng.standard_normal((10, 2, 16, 4)).astype(np.float32)
    ks = rng.random((10, 2)).astype(np.float32)
    vs = rng.random((10, 2)).astype(np.float32)
    pairs = [(1, 7), (1, 8), (4, 2)]
    k2, v2, ks2, vs2 = C.copy_blocks(kc, vc, pairs, ks, vs)
    for src, dst in pairs:
        assert np.array_equal(k2[dst], kc[src]) and np.array_equal(v2[dst], vc[src])
        assert np.array_equal(ks2[dst], ks[src]) and np.array_equal(vs2[dst], vs[src])
    for b in (0, 1, 3, 4, 5, 6, 9):
        assert np.array_equal(k2[b], kc[b]) and np.array_equal(v2[b], vc[b])


def test_parent_output_unchanged_by_children_copy_on_write():
    rng = np.random.default_rng(2)
    H, D, bs = 2, 16, 16
    bm = BlockManagerModel(24, bs, list(rng.permutation(24)))
    kc = np.full((24, H, bs, D), np.nan, np.float32)
    vc = np.full_like(kc, np.nan)
    parent = bm.seq_create(37)
    pk = rng.standard_normal((37, H, D)).astype(np.float32)
    pv = rng.standard_normal((37, H, D)).astype(np.float32)
    kc, vc = C.reshape_and_cache(pk, pv, kc, vc, bm.seq_slots(parent, 0, 37), bs)
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    t0, l0 = bm.export([parent], 4)
    before = A.decode(q, kc, vc, t0, l0, np.float32(0.25))
    kids = [bm.seq_fork(parent) for _ in range(3)]
    slots, cows = bm.seq_append_batch(kids)
    assert len(cows) == 3                      # the tail (5 of 16 filled) is shared
    kc, vc, _, _ = C.copy_blocks(kc, vc, cows)
    nk = rng.standard_normal((3, H, D)).astype(np.float32)
    kc, vc = C.reshape_and_cache(nk, nk, kc, vc, slots, bs)
    t1, l1 = bm.export([parent], 4)
    after = A.decode(q, kc, vc, t1, l1, np.float32(0.25))
    assert np.array_equal(t0, t1) and np.array_equal(before, after)
    # each child sees the parent's 37 rows plus its own new row
    tk, lk = bm.export(kids, 4)
    for i in range(3):
        K = A.gather(kc, tk[i], lk[i], bs)
        assert np.array_equal(K[:37], pk.astype(np.float64))
        assert np.array_equal(K[37], nk[i].astype(np.float64))


def test_swap_blocks_round_trip_and_untouched_blocks():
    rng = np.random.default_rng(5)
    dev_k = rng.standard_normal((12, 2, 16, 4)).astype(np.float32)
    dev_v = rng.standard_normal((12, 2, 16, 4)).astype(np.float32)
    host_k = np.full((5, 2, 16, 4), np.nan, np.float32)
    host_v = host_k.copy()
    out = [(7, 0), (2, 1), (11, 4)]               # device block -> host block
    hk, hv, _, _ = C.swap_blocks(host_k, host_v, dev_k, dev_v, out)
    for s, d in out:
        assert np.array_equal(hk[d], dev_k[s]) and np.array_equal(hv[d], dev_v[s])
    assert np.isnan(hk[[2, 3]]).all()             # host blocks not named stay as they were
    # swap back into other device blocks: the rows come back bit for bit
    back = [(0, 3), (1, 9), (4, 5)]
    nk = np.zeros_like(dev_k)
    nv = np.zeros_like(dev_v)
    k2, v2, _, _ = C.swap_blocks(nk, nv, hk, hv, back)
    for (s_dev, h), (h2, d_new) in zip(out, back):
        assert h == h2
        assert np.array_equal(k2[d_new], dev_k[s_dev]) and np.array_equal(v2[d_new], dev_v[s_dev])
    assert not k2[[0, 1, 2, 4, 6, 7, 8, 10, 11]].any()


def test_swap_blocks_scales_hand_worked():
    """The scale branch of swap_blocks, worked by hand: each (src, dst) pair
    moves src's K scales into dst's K scales and src's V scales into dst's V
    scales (never crossed), and destination blocks no pair names keep
    theirs.  Source pools: 3 blocks x 2 KV heads; destination: 4 blocks."""
    src_k = np.arange(3 * 2 * 16 * 2, dtype=np.float32).reshape(3, 2, 16, 2)
    src_v = -src_k
    src_ks = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]], np.float32)
    src_vs = np.array([[10.0, 20.0], [30.0, 40.0], [50.0, 60.0]], np.float32)
    dst_k = np.zeros((4, 2, 16, 2), np.float32)
    dst_v = np.zeros_like(dst_k)
    dst_ks = np.full((4, 2), -1.0, np.float32)
    dst_vs = np.full((4, 2), -2.0, np.float32)
    dk, dv, dks, dvs = C.swap_blocks(dst_k, dst_v, src_k, src_v, [(2, 0), (0, 3)],
                                     dst_ks, dst_vs, src_ks, src_vs)
    assert np.array_equal(dks, np.array([[5.0, 6.0], [-1.0, -1.0], [-1.0, -1.0], [1.0, 2.0]],
                                        np.float32))
    assert np.array_equal(dvs, np.array([[50.0, 60.0], [-2.0, -2.0], [-2.0, -2.0],
                                         [10.0, 20.0]], np.float32))
    assert np.array_equal(dk[0], src_k[2]) and np.array_equal(dv[3], src_v[0])
    assert not dk[[1, 2]].any() and not dv[[1, 2]].any()
    # the inputs are not modified
    assert (dst_ks == -1.0).all() and (dst_vs == -2.0).all()
