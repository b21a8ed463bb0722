"""GPU parity with every block past the 4 GiB mark of its pool.

A pool sized for a large share of the GPU's 288 GB puts block ids past
2^31 / 2^32 bytes of offset.  Each test takes a small seeded case, copies
its pool behind OFF empty blocks of a large device pool, shifts its block
table (and slots, and copy pairs) by OFF, and runs the same call on both
pools: the results are the same bits (only the addresses differ; the load
policy, which the pool size changes, changes no bit), and within the
attention tolerance of the oracle.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_366_amd as pkv
from oracle import attention as A
from oracle import cache_ops as C
from synth import workloads as W

from gpu_common import DEV, i32, out_f64, to_dev

pytestmark = pytest.mark.gpu

TOL16 = 2e-3
WAVE, MFMA = pkv.PKV_ALGO_WAVE, pkv.PKV_ALGO_MFMA
HQ, HKV, D, BS = 16, 8, 128, 16
LENS = [1, 17, 300, 1500, 3001]
# empty blocks ahead of the case's own: 4.59e9 bytes of bf16 blocks (32 KiB
# each), 4.59e9 bytes of int8 blocks (16 KiB each); both past 2^32
OFF16 = 140_000
OFF8 = 280_000


def big(small: torch.Tensor, off: int) -> torch.Tensor:
    t = torch.zeros((off + small.shape[0],) + tuple(small.shape[1:]), dtype=small.dtype,
                    device=DEV)
    t[off:] = small
    return t


def shift(tables: np.ndarray, off: int) -> torch.Tensor:
    return i32(np.where(tables >= 0, tables + off, -1))


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_offsets_pass_4_gib():
    assert OFF16 * HKV * BS * D * 2 > 2 ** 32 and OFF8 * HKV * BS * D > 2 ** 32


@pytest.mark.parametrize("algo", [WAVE, MFMA], ids=["wave", "mfma"])
def test_decode_bf16(algo):
    c = W.decode_case(900, len(LENS), HQ, HKV, D, lens=LENS, dtype="bf16")
    q = to_dev(c.q, "bf16")
    k, v = to_dev(c.k_cache, "bf16"), to_dev(c.v_cache, "bf16")
    kb, vb = big(k, OFF16), big(v, OFF16)
    ref = A.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale)
    mx = int(c.context_lens.max())
    for parts in (0, 256):
        o_s = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        o_b = torch.empty_like(o_s)
        pkv.pkv_paged_attention_decode(o_s, q, k, v, i32(c.block_tables), i32(c.context_lens), mx,
                                       float(c.scale), parts, algo)
        pkv.pkv_paged_attention_decode(o_b, q, kb, vb, shift(c.block_tables, OFF16),
                                       i32(c.context_lens), mx, float(c.scale), parts, algo)
        torch.cuda.synchronize()
        assert torch.equal(o_b, o_s), parts
        assert np.abs(out_f64(o_b) - ref).max() <= TOL16
    del kb, vb
    free()


@pytest.mark.parametrize("algo", [WAVE, MFMA], ids=["wave", "mfma"])
def test_decode_int8(algo):
    c = W.decode_case(901, len(LENS), HQ, HKV, D, lens=LENS, dtype="bf16", int8=True)
    q = to_dev(c.q, "bf16")
    k, v = torch.from_numpy(c.k_i8).to(DEV), torch.from_numpy(c.v_i8).to(DEV)
    ks, vs = torch.from_numpy(c.k_scale).to(DEV), torch.from_numpy(c.v_scale).to(DEV)
    kb, vb, ksb, vsb = big(k, OFF8), big(v, OFF8), big(ks, OFF8), big(vs, OFF8)
    ref = A.decode(c.q, c.k_i8, c.v_i8, c.block_tables, c.context_lens, c.scale,
                   k_scale=c.k_scale, v_scale=c.v_scale)
    mx = int(c.context_lens.max())
    for parts in (0, 256):
        o_s = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        o_b = torch.empty_like(o_s)
        pkv.pkv_paged_attention_decode(o_s, q, k, v, i32(c.block_tables), i32(c.context_lens), mx,
                                       float(c.scale), parts, algo, ks, vs)
        pkv.pkv_paged_attention_decode(o_b, q, kb, vb, shift(c.block_tables, OFF8),
                                       i32(c.context_lens), mx, float(c.scale), parts, algo,
                                       ksb, vsb)
        torch.cuda.synchronize()
        assert torch.equal(o_b, o_s), parts
        assert np.abs(out_f64(o_b) - ref).max() <= TOL16
    del kb, vb
    free()


def test_decode_step_appends_past_4_gib():
    """The one-launch step writes each sequence's new rows into its last
    block (past 4 GiB) and attends them."""
    c = W.decode_case(902, len(LENS), HQ, HKV, D, lens=LENS, dtype="bf16")
    q = to_dev(c.q, "bf16")
    rng = np.random.default_rng(3)
    nk = to_dev(W.draw_normal(rng, (len(LENS), HKV, D), "bf16"), "bf16")
    nv = to_dev(W.draw_normal(rng, (len(LENS), HKV, D), "bf16"), "bf16")
    k, v = to_dev(c.k_cache, "bf16"), to_dev(c.v_cache, "bf16")
    kb, vb = big(k, OFF16), big(v, OFF16)
    mx = int(c.context_lens.max())
    for algo in (WAVE, MFMA):
        o_s = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        o_b = torch.empty_like(o_s)
        pkv.pkv_paged_attention_decode_step(o_s, q, nk, nv, k, v, i32(c.block_tables),
                                            i32(c.context_lens), mx, float(c.scale), 256, algo)
        pkv.pkv_paged_attention_decode_step(o_b, q, nk, nv, kb, vb, shift(c.block_tables, OFF16),
                                            i32(c.context_lens), mx, float(c.scale), 256, algo)
        torch.cuda.synchronize()
        assert torch.equal(o_b, o_s), algo
        # bit for bit (the pool holds NaN in its unwritten slots)
        assert torch.equal(kb[OFF16:].view(torch.int16), k.view(torch.int16)), algo
        assert torch.equal(vb[OFF16:].view(torch.int16), v.view(torch.int16)), algo
        assert not kb[:OFF16].any().item() and not vb[:OFF16].any().item()
    del kb, vb
    free()


def test_prefill():
    chunks = [(0, 70), (300, 130), (1500, 64), (777, 1)]
    c = W.prefill_case(903, HQ, HKV, D, chunks, dtype="bf16")
    q = to_dev(c.q, "bf16")
    k, v = to_dev(c.k_cache, "bf16"), to_dev(c.v_cache, "bf16")
    kb, vb = big(k, OFF16), big(v, OFF16)
    ref = A.prefill(c.q, c.k_cache, c.v_cache, c.block_tables, c.query_start_loc,
                    c.context_lens, c.scale)
    max_q = int(np.diff(c.query_start_loc).max())
    mx = int(c.context_lens.max())
    for parts in (0, 256):
        o_s = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        o_b = torch.empty_like(o_s)
        pkv.pkv_paged_attention_prefill(o_s, q, k, v, i32(c.block_tables), i32(c.query_start_loc),
                                        i32(c.context_lens), max_q, mx, float(c.scale),
                                        partition_tokens=parts)
        pkv.pkv_paged_attention_prefill(o_b, q, kb, vb, shift(c.block_tables, OFF16),
                                        i32(c.query_start_loc), i32(c.context_lens), max_q, mx,
                                        float(c.scale), partition_tokens=parts)
        torch.cuda.synchronize()
        assert torch.equal(o_b, o_s), parts
        assert np.abs(out_f64(o_b) - ref).max() <= TOL16
    del kb, vb
    free()


def test_reshape_and_cache_and_copy_blocks():
    rng = np.random.default_rng(904)
    nb = 40
    pk = W.draw_normal(rng, (nb, HKV, BS, D), "bf16")
    pv = W.draw_normal(rng, (nb, HKV, BS, D), "bf16")
    small_k, small_v = to_dev(pk, "bf16"), to_dev(pv, "bf16")
    kb, vb = big(small_k, OFF16), big(small_v, OFF16)
    T = 50
    slots = rng.choice(nb * BS, T, replace=False).astype(np.int32)
    slots[::7] = -1
    nk = W.draw_normal(rng, (T, HKV, D), "bf16")
    nv = W.draw_normal(rng, (T, HKV, D), "bf16")
    key, val = to_dev(nk, "bf16"), to_dev(nv, "bf16")
    pkv.pkv_reshape_and_cache(key, val, small_k, small_v, i32(slots))
    pkv.pkv_reshape_and_cache(key, val, kb, vb, i32(np.where(slots >= 0, slots + OFF16 * BS, -1)))
    pairs = np.array([[3, 30], [17, 5], [0, 39], [22, 23]], np.int32)
    pkv.pkv_copy_blocks(small_k, small_v, i32(pairs))
    pkv.pkv_copy_blocks(kb, vb, i32(pairs + OFF16))
    torch.cuda.synchronize()
    assert torch.equal(kb[OFF16:], small_k) and torch.equal(vb[OFF16:], small_v)
    assert not kb[:OFF16].any().item() and not vb[:OFF16].any().item()
    # both against the plain definitions: the rows written, then the copies
    ek, ev = C.reshape_and_cache(nk, nv, pk, pv, slots, BS)
    ek, ev, _, _ = C.copy_blocks(ek, ev, pairs)
    assert np.array_equal(kb[OFF16:].float().cpu().numpy(), ek)
    assert np.array_equal(vb[OFF16:].float().cpu().numpy(), ev)
    del kb, vb
    free()


def test_int8_encoder_quantised_writes_and_swaps():
    """The block encoder, quantise-on-write and swaps to and from a pinned
    host pool, with the device blocks past 4 GiB of int8 codes (and 9 GB of
    bf16 source blocks)."""
    rng = np.random.default_rng(905)
    nb = 40
    pk = W.draw_normal(rng, (nb, HKV, BS, D), "bf16")
    pv = W.draw_normal(rng, (nb, HKV, BS, D), "bf16")
    sk, sv = to_dev(pk, "bf16"), to_dev(pv, "bf16")
    skb, svb = big(sk, OFF8), big(sv, OFF8)
    codes = lambda n: torch.zeros((n, HKV, BS, D), dtype=torch.int8, device=DEV)
    scales = lambda n: torch.zeros((n, HKV), dtype=torch.float32, device=DEV)
    dk, dv, ks, vs = codes(nb), codes(nb), scales(nb), scales(nb)
    dkb, dvb, ksb, vsb = codes(OFF8 + nb), codes(OFF8 + nb), scales(OFF8 + nb), scales(OFF8 + nb)
    blocks = np.array([3, 17, 0, 39, 22], np.int32)
    filled = np.array([16, 1, 9, 16, 5], np.int32)
    pkv.pkv_quantize_blocks(sk, sv, dk, dv, ks, vs, i32(blocks), i32(filled))
    pkv.pkv_quantize_blocks(skb, svb, dkb, dvb, ksb, vsb, i32(blocks + OFF8), i32(filled))
    del skb, svb
    # quantise-on-write: a run continuing block 0 (filled 9), a new block
    T = 6
    slots = np.array([9, 10, 11, 5 * BS, 5 * BS + 1, 22 * BS + 5], np.int32)
    nk = to_dev(W.draw_normal(rng, (T, HKV, D), "bf16"), "bf16")
    nv = to_dev(W.draw_normal(rng, (T, HKV, D), "bf16"), "bf16")
    pkv.pkv_reshape_and_cache_int8(nk, nv, dk, dv, ks, vs, i32(slots))
    pkv.pkv_reshape_and_cache_int8(nk, nv, dkb, dvb, ksb, vsb, i32(slots + OFF8 * BS))
    torch.cuda.synchronize()
    assert torch.equal(dkb[OFF8:], dk) and torch.equal(dvb[OFF8:], dv)
    assert torch.equal(ksb[OFF8:].view(torch.int32), ks.view(torch.int32))
    assert torch.equal(vsb[OFF8:].view(torch.int32), vs.view(torch.int32))
    assert not dkb[:OFF8].any().item() and not ksb[:OFF8].any().item()
    # swap out to a pinned host pool, then back into other device blocks
    hk = torch.zeros((8, HKV, BS, D), dtype=torch.int8, pin_memory=True)
    hv = torch.zeros((8, HKV, BS, D), dtype=torch.int8, pin_memory=True)
    hks = torch.zeros((8, HKV), dtype=torch.float32, pin_memory=True)
    hvs = torch.zeros((8, HKV), dtype=torch.float32, pin_memory=True)
    out_pairs = np.array([[3, 0], [17, 1], [22, 2], [0, 7]], np.int32)
    pkv.pkv_swap_blocks(hk, hv, dkb, dvb, out_pairs + [OFF8, 0], hks, hvs, ksb, vsb)
    torch.cuda.synchronize()
    assert torch.equal(hk[[0, 1, 2, 7]], dk[[3, 17, 22, 0]].cpu())
    assert torch.equal(hks[[0, 1, 2, 7]].view(torch.int32), ks[[3, 17, 22, 0]].cpu().view(torch.int32))
    in_pairs = np.array([[0, 30], [1, 31], [7, 35]], np.int32)
    pkv.pkv_swap_blocks(dkb, dvb, hk, hv, in_pairs + [0, OFF8], ksb, vsb, hks, hvs)
    torch.cuda.synchronize()
    assert torch.equal(dkb[OFF8 + 30], dk[3]) and torch.equal(dvb[OFF8 + 31], dv[17])
    assert torch.equal(dkb[OFF8 + 35], dk[0]) and ksb[OFF8 + 31, 0].item() == ks[17, 0].item()
    del dkb, dvb
    free()
