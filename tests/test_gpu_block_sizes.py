"""GPU parity at block sizes 32, 64 and 128 (the kernels walk every block as
16-row tiles).  Decode and prefill against the float64 oracle at the same
block size, with ragged lengths around block edges; the same logical K/V laid
out in 16-row and in larger blocks give bit-identical outputs (the kernels'
arithmetic and order do not depend on the block size); cache writes, block
copies, int8 encoding and swaps bit-exact; and a whole step through the
block manager at block size 64."""
import functools

import numpy as np
import pytest
import torch

import paged_kv_cache_366_amd as pkv
from oracle import attention as A
from oracle import cache_ops as C
from oracle import quantize as Q
from synth import workloads as W

from gpu_common import DEV, TORCH_DT, i32, out_f64, to_dev

pytestmark = pytest.mark.gpu
TOL16, TOL32 = 2e-3, 1e-5
WAVE, MFMA = pkv.PKV_ALGO_WAVE, pkv.PKV_ALGO_MFMA
SIZES = [32, 64, 128]

# (q heads, kv heads, head_dim, dtype, algo, int8)
KINDS = {
    "mha-bf16-wave": (8, 8, 128, "bf16", WAVE, False),
    "gqa-bf16-mfma": (16, 2, 128, "bf16", MFMA, False),
    "gqa-int8-mfma": (16, 2, 128, "bf16", MFMA, True),
    "mha-int8-wave": (8, 8, 128, "bf16", WAVE, True),
    "mha-f16-wave-d64": (4, 4, 64, "f16", WAVE, False),
    "gqa-f32-wave-d64": (4, 2, 64, "f32", WAVE, False),
}


def lens_for(bs):
    # one token, around one block edge, around two, several blocks, long
    return [1, bs - 1, bs, bs + 1, 2 * bs - 1, 2 * bs + 1, 300, 777, 1500, 16]


@functools.lru_cache(maxsize=None)
def decode_case(kind, bs):
    hq, hkv, d, dtype, _, int8 = KINDS[kind]
    c = W.decode_case(900 + bs, 10, hq, hkv, d, lens=lens_for(bs), dtype=dtype, block_size=bs,
                      int8=int8, keep_logical=True)
    if int8:
        ref = A.decode(c.q, c.k_i8, c.v_i8, c.block_tables, c.context_lens, c.scale,
                       block_size=bs, k_scale=c.k_scale, v_scale=c.v_scale)
    else:
        ref = A.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale,
                       block_size=bs)
    return c, ref


def run_decode(c, algo, parts, int8=False, k=None, v=None, tables=None):
    q = to_dev(c.q, c.dtype)
    if int8:
        k = torch.from_numpy(c.k_i8).to(DEV) if k is None else k
        v = torch.from_numpy(c.v_i8).to(DEV) if v is None else v
        ks, vs = torch.from_numpy(c.k_scale).to(DEV), torch.from_numpy(c.v_scale).to(DEV)
    else:
        k = to_dev(c.k_cache, c.dtype) if k is None else k
        v = to_dev(c.v_cache, c.dtype) if v is None else v
        ks = vs = None
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    pkv.pkv_paged_attention_decode(out, q, k, v, i32(c.block_tables if tables is None else tables),
                                   i32(c.context_lens), int(c.context_lens.max()),
                                   float(c.scale), parts, algo, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("parts", [0, 16, 256])
@pytest.mark.parametrize("bs", SIZES)
@pytest.mark.parametrize("kind", list(KINDS))
def test_decode_matches_oracle(kind, bs, parts):
    c, ref = decode_case(kind, bs)
    _, _, _, dtype, algo, int8 = KINDS[kind]
    out = run_decode(c, algo, parts, int8)
    err = np.abs(out_f64(out) - ref).max()
    assert err <= (TOL32 if dtype == "f32" else TOL16), (kind, bs, parts, err)


def relaid(c, bs, seed):
    """The logical K/V of a 16-row-block case laid out in blocks of ``bs``."""
    lens = c.context_lens
    nb = W.pool_size(lens, 1.25, bs)
    perm = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    tables = W.place_by_permutation(lens, perm, bs)
    shape = (nb, c.kv_heads, bs, c.head_dim)
    kc = np.full(shape, np.nan, np.float32)
    vc = kc.copy()
    for s in range(len(lens)):
        W.scatter_rows(kc, tables[s], c.k_logical[s], bs)
        W.scatter_rows(vc, tables[s], c.v_logical[s], bs)
    return kc, vc, tables


@pytest.mark.parametrize("algo", [WAVE, MFMA], ids=["wave", "mfma"])
@pytest.mark.parametrize("parts", [0, 48, 512])
def test_decode_bits_do_not_depend_on_block_size(algo, parts):
    c = W.decode_case(77, 9, 8, 2, 128, len_range=(1, 1200), dtype="bf16", keep_logical=True)
    base = run_decode(c, algo, parts)
    for bs in SIZES:
        kc, vc, tables = relaid(c, bs, bs)
        out = run_decode(c, algo, parts, k=to_dev(kc, "bf16"), v=to_dev(vc, "bf16"),
                         tables=tables)
        assert torch.equal(out, base), (bs, (out - base).abs().max().item())


CHUNKS = [(0, 1), (0, 17), (7, 64), (16, 65), (100, 130), (33, 0), (250, 16), (5, 3), (127, 129)]


@pytest.mark.parametrize("bs", SIZES)
@pytest.mark.parametrize("hq,hkv,d,dtype", [(8, 2, 128, "bf16"), (4, 4, 64, "f16"),
                                            (4, 2, 64, "f32")])
def test_prefill_matches_oracle_and_is_block_size_blind(bs, hq, hkv, d, dtype):
    c = W.prefill_case(600 + bs, hq, hkv, d, CHUNKS, dtype=dtype, block_size=bs,
                       keep_logical=True)
    ref = A.prefill(c.q, c.k_cache, c.v_cache, c.block_tables, c.query_start_loc,
                    c.context_lens, c.scale, block_size=bs)

    def run(kc, vc, tables):
        qd = to_dev(c.q, dtype)
        out = torch.empty(qd.shape, dtype=torch.float32, device=DEV)
        pkv.pkv_paged_attention_prefill(out, qd, to_dev(kc, dtype), to_dev(vc, dtype), i32(tables),
                                        i32(c.query_start_loc), i32(c.context_lens),
                                        int(np.diff(c.query_start_loc).max()),
                                        int(c.context_lens.max()), float(c.scale))
        torch.cuda.synchronize()
        return out

    out = run(c.k_cache, c.v_cache, c.block_tables)
    err = np.abs(out_f64(out) - ref).max()
    assert err <= (TOL32 if dtype == "f32" else TOL16), err
    # the same logical rows in 16-row blocks: bit-identical
    lens = c.context_lens
    nb16 = W.pool_size(lens, 1.25, 16)
    t16 = W.place_by_permutation(lens, np.random.default_rng(1).permutation(nb16), 16)
    k16 = np.full((nb16, hkv, 16, d), np.nan, np.float32)
    v16 = k16.copy()
    for s in range(len(lens)):
        W.scatter_rows(k16, t16[s], c.k_logical[s], 16)
        W.scatter_rows(v16, t16[s], c.v_logical[s], 16)
    assert torch.equal(run(k16, v16, t16.astype(np.int32)), out)


@pytest.mark.parametrize("bs", SIZES)
def test_cache_ops_bit_exact(bs):
    rng = np.random.default_rng(bs)
    nb, hkv, d, T = 12, 4, 128, 150
    kc = W.draw_normal(rng, (nb, hkv, bs, d), "bf16")
    vc = W.draw_normal(rng, (nb, hkv, bs, d), "bf16")
    key = W.draw_normal(rng, (T, hkv, d), "bf16")
    val = W.draw_normal(rng, (T, hkv, d), "bf16")
    slots = W.distinct_slots(rng, nb * bs, T, skip_fraction=0.1)
    rk, rv = C.reshape_and_cache(key, val, kc, vc, slots, bs)
    dk, dv = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    pkv.pkv_reshape_and_cache(to_dev(key, "bf16"), to_dev(val, "bf16"), dk, dv, i32(slots))
    torch.cuda.synchronize()
    assert np.array_equal(dk.float().cpu().numpy(), rk)
    assert np.array_equal(dv.float().cpu().numpy(), rv)
    # copy_blocks
    pairs = np.array([(1, 7), (1, 8), (4, 2), (11, 0)], np.int32)
    rk2, rv2, _, _ = C.copy_blocks(rk, rv, pairs)
    pkv.pkv_copy_blocks(dk, dv, i32(pairs))
    torch.cuda.synchronize()
    assert np.array_equal(dk.float().cpu().numpy(), rk2)
    assert np.array_equal(dv.float().cpu().numpy(), rv2)
    # int8 encoding of whole blocks, with filled counts up to the block size
    blocks = np.array([0, 3, 5, 9, 11], np.int32)
    filled = np.array([bs, 1, bs - 1, bs // 2 + 3, 0], np.int32)
    ck = torch.full((nb, hkv, bs, d), 55, dtype=torch.int8, device=DEV)
    cv = ck.clone()
    sk = torch.full((nb, hkv), 9.0, dtype=torch.float32, device=DEV)
    sv = sk.clone()
    pkv.pkv_quantize_blocks(dk, dv, ck, cv, sk, sv, i32(blocks), i32(filled))
    torch.cuda.synchronize()
    base_c = np.full((nb, hkv, bs, d), 55, np.int8)
    base_s = np.full((nb, hkv), 9.0, np.float32)
    ok, oks = Q.quantize_blocks(rk2, base_c, base_s, blocks, filled)
    ov, ovs = Q.quantize_blocks(rv2, base_c, base_s, blocks, filled)
    assert np.array_equal(ck.cpu().numpy(), ok) and np.array_equal(cv.cpu().numpy(), ov)
    assert np.array_equal(sk.cpu().numpy().view(np.uint32), oks.view(np.uint32))
    assert np.array_equal(sv.cpu().numpy().view(np.uint32), ovs.view(np.uint32))
    # swap out to pinned host memory and back into other blocks
    hk = torch.zeros((5, hkv, bs, d), dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    out_pairs = np.array([[2, 0], [3, 1], [7, 2], [10, 4]], np.int32)
    ws = torch.empty(pkv.pkv_swap_workspace_bytes(2, hkv, d, bs, pkv.PKV_BF16), dtype=torch.uint8,
                     device=DEV)
    pkv.pkv_swap_blocks(hk, hv, dk, dv, out_pairs, workspace=ws)
    torch.cuda.synchronize()
    z = np.zeros((5, hkv, bs, d), np.float32)
    rhk, rhv, _, _ = C.swap_blocks(z, z, rk2, rv2, out_pairs)
    assert np.array_equal(hk.float().numpy(), rhk) and np.array_equal(hv.float().numpy(), rhv)


def test_block_manager_step_at_block_size_64():
    bs, hq, hkv, d = 64, 8, 4, 128
    rng = np.random.default_rng(64)
    lens = np.array([1, 63, 64, 65, 200, 129, 700], np.int32)
    nb = W.pool_size(lens + 1, 1.5, bs)
    bm = pkv.pkv_bm_create(nb, bs, rng.permutation(nb).astype(np.int32))
    try:
        kc = np.full((nb, hkv, bs, d), np.nan, np.float32)
        vc = kc.copy()
        dk, dv = to_dev(kc, "bf16"), to_dev(vc, "bf16")
        sids = [pkv.pkv_seq_create(bm, 0) for _ in lens]
        # prompt rows through reshape_and_cache, then one decode token each
        for sid, n in zip(sids, lens):
            k = W.draw_normal(rng, (int(n), hkv, d), "bf16")
            v = W.draw_normal(rng, (int(n), hkv, d), "bf16")
            sl = pkv.pkv_seq_append(bm, sid, int(n))[0]
            kc, vc = C.reshape_and_cache(k, v, kc, vc, sl, bs)
            pkv.pkv_reshape_and_cache(to_dev(k, "bf16"), to_dev(v, "bf16"), dk, dv, i32(sl))
        slots, cow = pkv.pkv_seq_append_batch(bm, sids)
        assert len(cow) == 0
        nk = W.draw_normal(rng, (len(lens), hkv, d), "bf16")
        nv = W.draw_normal(rng, (len(lens), hkv, d), "bf16")
        kc, vc = C.reshape_and_cache(nk, nv, kc, vc, slots, bs)
        pkv.pkv_reshape_and_cache(to_dev(nk, "bf16"), to_dev(nv, "bf16"), dk, dv, i32(slots))
        tables, lens2 = pkv.pkv_seq_export(bm, sids, W.blocks_for(int(lens.max()) + 1, bs))
        q = W.draw_normal(rng, (len(lens), hq, d), "bf16")
        out = torch.empty((len(lens), hq, d), dtype=torch.float32, device=DEV)
        pkv.pkv_paged_attention_decode(out, to_dev(q, "bf16"), dk, dv, i32(tables), i32(lens2),
                                       int(lens2.max()), float(1 / np.sqrt(d)), 128)
        torch.cuda.synchronize()
        ref = A.decode(q, kc, vc, tables, lens2, np.float32(1 / np.sqrt(d)), block_size=bs)
        assert np.abs(out_f64(out) - ref).max() <= TOL16
        assert np.array_equal(dk.float().cpu().numpy()[~np.isnan(kc)], kc[~np.isnan(kc)])
    finally:
        pkv.pkv_bm_destroy(bm)
