"""GPU parity of swap_blocks (device <-> pinned host pools) against the
oracle: bit-exact copies, untouched blocks unchanged, int8 scales carried,
and decode after a swap-out / swap-in round trip bit-identical to decode
before it (attention does not depend on where blocks sit)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_366_amd as pkv
from oracle import cache_ops as C
from synth import workloads as W

from gpu_common import DEV, i32, to_dev

pytestmark = pytest.mark.gpu


def host_pool(shape, dtype, fill=0):
    return torch.full(shape, fill, dtype=dtype).pin_memory()


def workspace(kind, hkv, d, dtype_code=pkv.PKV_BF16):
    """None (one DMA copy per run), room for 3 blocks (several rounds), or all."""
    if kind is None:
        return None
    n = 3 if kind == "small" else 64
    return torch.empty(pkv.pkv_swap_workspace_bytes(n, hkv, d, 16, dtype_code), dtype=torch.uint8,
                       device=DEV)


@pytest.mark.parametrize("ws", [None, "small", "large"])
def test_device_to_host_to_device_bit_exact(ws):
    rng = np.random.default_rng(20)
    nb, hkv, d = 24, 4, 128
    kc = W.draw_normal(rng, (nb, hkv, 16, d), "bf16")
    vc = W.draw_normal(rng, (nb, hkv, 16, d), "bf16")
    dk, dv = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    hk = host_pool((10, hkv, 16, d), torch.bfloat16, 7.0)
    hv = host_pool((10, hkv, 16, d), torch.bfloat16, 7.0)
    out = np.array([[5, 0], [6, 1], [7, 2], [20, 5], [1, 9], [2, 8]], np.int32)  # runs and singles
    w = workspace(ws, hkv, d)
    pkv.pkv_swap_blocks(hk, hv, dk, dv, out, workspace=w)
    torch.cuda.synchronize()
    ref_hk, ref_hv, _, _ = C.swap_blocks(np.full((10, hkv, 16, d), 7.0, np.float32),
                                         np.full((10, hkv, 16, d), 7.0, np.float32), kc, vc, out)
    assert np.array_equal(hk.float().numpy(), ref_hk) and np.array_equal(hv.float().numpy(), ref_hv)
    # back into different device blocks of a fresh pool
    nk = torch.zeros((nb, hkv, 16, d), dtype=torch.bfloat16, device=DEV)
    nv = torch.zeros_like(nk)
    back = np.array([[0, 11], [1, 12], [2, 13], [5, 3], [9, 23], [8, 0]], np.int32)
    pkv.pkv_swap_blocks(nk, nv, hk, hv, back, workspace=w)
    torch.cuda.synchronize()
    ref_k, ref_v, _, _ = C.swap_blocks(np.zeros((nb, hkv, 16, d), np.float32),
                                       np.zeros((nb, hkv, 16, d), np.float32), ref_hk, ref_hv, back)
    assert np.array_equal(nk.float().cpu().numpy(), ref_k)
    assert np.array_equal(nv.float().cpu().numpy(), ref_v)


@pytest.mark.parametrize("ws", [None, "large"])
def test_device_to_device(ws):
    rng = np.random.default_rng(23)
    nb, hkv, d = 16, 2, 64
    kc = W.draw_normal(rng, (nb, hkv, 16, d), "f16")
    vc = W.draw_normal(rng, (nb, hkv, 16, d), "f16")
    dk, dv = to_dev(kc, "f16"), to_dev(vc, "f16")
    ok = torch.full((6, hkv, 16, d), -1.0, dtype=torch.float16, device=DEV)
    ov = ok.clone()
    pairs = np.array([[15, 0], [3, 5], [4, 2]], np.int32)
    pkv.pkv_swap_blocks(ok, ov, dk, dv, pairs, workspace=workspace(ws, hkv, d, pkv.PKV_F16))
    torch.cuda.synchronize()
    rk, rv, _, _ = C.swap_blocks(np.full((6, hkv, 16, d), -1.0, np.float32),
                                 np.full((6, hkv, 16, d), -1.0, np.float32), kc, vc, pairs)
    assert np.array_equal(ok.float().cpu().numpy(), rk)
    assert np.array_equal(ov.float().cpu().numpy(), rv)


@pytest.mark.parametrize("ws", [None, "small"])
def test_int8_pool_with_scales(ws):
    rng = np.random.default_rng(21)
    nb, hkv, d = 8, 2, 64
    codes = rng.integers(-127, 128, (nb, hkv, 16, d), dtype=np.int8)
    scales = rng.random((nb, hkv)).astype(np.float32)
    dk, dv = torch.from_numpy(codes).to(DEV), torch.from_numpy(codes[::-1].copy()).to(DEV)
    ks, vs = torch.from_numpy(scales).to(DEV), torch.from_numpy(scales[::-1].copy()).to(DEV)
    hk = host_pool((4, hkv, 16, d), torch.int8)
    hv = host_pool((4, hkv, 16, d), torch.int8)
    hks = host_pool((4, hkv), torch.float32)
    hvs = host_pool((4, hkv), torch.float32)
    pairs = np.array([[3, 0], [4, 1], [0, 3]], np.int32)
    pkv.pkv_swap_blocks(hk, hv, dk, dv, pairs, hks, hvs, ks, vs,
                        workspace=workspace(ws, hkv, d, pkv.PKV_I8))
    torch.cuda.synchronize()
    rk, rv, rks, rvs = C.swap_blocks(np.zeros((4, hkv, 16, d), np.int8), np.zeros((4, hkv, 16, d), np.int8),
                                     codes, codes[::-1].copy(), pairs, np.zeros((4, hkv), np.float32),
                                     np.zeros((4, hkv), np.float32), scales, scales[::-1].copy())
    assert np.array_equal(hk.numpy(), rk) and np.array_equal(hv.numpy(), rv)
    assert np.array_equal(hks.numpy().view(np.uint32), rks.view(np.uint32))
    assert np.array_equal(hvs.numpy().view(np.uint32), rvs.view(np.uint32))


def test_decode_after_swap_round_trip_is_bit_identical():
    c = W.decode_case(22, 6, 8, 8, 128, lens=[40, 300, 17, 128, 511, 2], dtype="bf16",
                      pool_factor=2.5)
    dk, dv = to_dev(c.k_cache, "bf16"), to_dev(c.v_cache, "bf16")
    q = to_dev(c.q, "bf16")
    mc = int(c.context_lens.max())

    def decode(tables):
        out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        pkv.pkv_paged_attention_decode(out, q, dk, dv, i32(tables), i32(c.context_lens), mc,
                                       float(c.scale), 128)
        torch.cuda.synchronize()
        return out.clone()

    before = decode(c.block_tables)
    # preempt sequence 4: its blocks go to host memory, its device blocks are
    # overwritten by other data, then it resumes in different device blocks
    s = 4
    nblk = W.blocks_for(c.context_lens[s])
    own = c.block_tables[s, :nblk].copy()
    hk = host_pool((nblk,) + tuple(dk.shape[1:]), torch.bfloat16)
    hv = host_pool((nblk,) + tuple(dk.shape[1:]), torch.bfloat16)
    w = workspace("small", dk.shape[1], dk.shape[3])
    pkv.pkv_swap_blocks(hk, hv, dk, dv, np.stack([own, np.arange(nblk)], 1), workspace=w)
    torch.cuda.synchronize()
    dk[torch.from_numpy(own.astype(np.int64)).to(DEV)] = 3.0
    dv[torch.from_numpy(own.astype(np.int64)).to(DEV)] = -3.0
    used = set(int(b) for b in c.block_tables[c.block_tables >= 0])
    free = np.array([b for b in range(c.num_blocks) if b not in used][:nblk], np.int32)
    assert len(free) == nblk
    pkv.pkv_swap_blocks(dk, dv, hk, hv, np.stack([np.arange(nblk), free], 1), workspace=w)
    tables = c.block_tables.copy()
    tables[s, :nblk] = free
    after = decode(tables)
    assert torch.equal(before, after)


def test_swap_counters_count_blocks_and_bytes():
    pkv.pkv_swap_stats_get(reset=True)
    nb, hkv, d = 12, 2, 64
    dk = torch.zeros((nb, hkv, 16, d), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    hk = host_pool((6, hkv, 16, d), torch.bfloat16)
    hv = host_pool((6, hkv, 16, d), torch.bfloat16)
    ws = workspace("large", hkv, d)
    pkv.pkv_swap_blocks(hk, hv, dk, dv, np.array([[0, 0], [3, 1], [4, 2]], np.int32), workspace=ws)
    pkv.pkv_swap_blocks(dk, dv, hk, hv, np.array([[0, 5], [1, 6]], np.int32), workspace=ws)
    pkv.pkv_swap_blocks(dk, dv, dk, dv, np.array([[7, 8]], np.int32), workspace=ws)
    torch.cuda.synchronize()
    st = pkv.pkv_swap_stats_get(reset=True)
    block = hkv * 16 * d * 2
    assert st == {"calls": 3, "blocks_to_host": 3, "blocks_to_device": 2,
                  "blocks_device_to_device": 1, "blocks_host_to_host": 0,
                  "bytes": 6 * 2 * block}
    assert pkv.pkv_swap_stats_get()["calls"] == 0
