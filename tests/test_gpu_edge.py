"""Edge cases of the device entry points: empty calls, batches whose every
context is empty, and contexts that fill their block-table row exactly
(split into the smallest and the largest partitions)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_366_amd as pkv
from oracle import attention as A
from synth import workloads as W

from gpu_common import DEV, DevCase, i32, out_f64, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


def snapshot(*ts):
    return [t.clone() for t in ts]


def unchanged(before, after):
    # compare bytes, so NaN patterns count as equal
    return all(torch.equal(b.view(torch.uint8), a.view(torch.uint8)) for b, a in zip(before, after))


def test_zero_size_calls_leave_everything_unchanged():
    rng = np.random.default_rng(70)
    nb, hkv, bs, d = 8, 2, 16, 64
    kc = to_dev(W.draw_normal(rng, (nb, hkv, bs, d), "bf16"), "bf16")
    vc = to_dev(W.draw_normal(rng, (nb, hkv, bs, d), "bf16"), "bf16")
    k8 = torch.from_numpy(rng.integers(-127, 128, (nb, hkv, bs, d), dtype=np.int8)).to(DEV)
    v8 = k8.flip(0).contiguous()
    k4 = torch.from_numpy(rng.integers(0, 256, (nb, hkv, bs, d // 2), dtype=np.uint8)).to(DEV)
    v4 = k4.flip(0).contiguous()
    ks = torch.rand((nb, hkv), device=DEV) + 0.1
    vs = torch.rand((nb, hkv), device=DEV) + 0.1
    state = snapshot(kc, vc, k8, v8, k4, v4, ks, vs)

    no_rows = torch.empty((0, hkv, d), dtype=torch.bfloat16, device=DEV)
    no_slots = torch.empty((0,), dtype=torch.int32, device=DEV)
    pkv.pkv_reshape_and_cache(no_rows, no_rows, kc, vc, no_slots)
    pkv.pkv_reshape_and_cache_int8(no_rows, no_rows, k8, v8, ks, vs, no_slots)
    pkv.pkv_reshape_and_cache_int4(no_rows, no_rows, k4, v4, ks, vs, no_slots)
    no_pairs = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    pkv.pkv_copy_blocks(kc, vc, no_pairs)
    pkv.pkv_copy_blocks(k8, v8, no_pairs, ks, vs)
    pkv.pkv_quantize_blocks(kc, vc, k8, v8, ks, vs, no_slots, no_slots)
    pkv.pkv_quantize_blocks_int4(kc, vc, k4, v4, ks, vs, no_slots, no_slots)
    pkv.pkv_swap_blocks(kc, vc, vc.clone(), kc.clone(), np.zeros((0, 2), np.int32))

    # no sequences at all
    q0 = torch.empty((0, 4, d), dtype=torch.bfloat16, device=DEV)
    out0 = torch.empty((0, 4, d), dtype=torch.float32, device=DEV)
    tables0 = torch.empty((0, 3), dtype=torch.int32, device=DEV)
    for algo in (pkv.PKV_ALGO_WAVE, pkv.PKV_ALGO_MFMA):
        for parts in (0, 16):
            pkv.pkv_paged_attention_decode(out0, q0, kc, vc, tables0, no_slots, 48, 0.125, parts,
                                           algo)
    # prefill with no query rows: no sequences, and sequences whose chunks are empty
    pkv.pkv_paged_attention_prefill(out0, q0, kc, vc, tables0, i32([0]), no_slots, 0, 48, 0.125)
    pkv.pkv_paged_attention_prefill(out0, q0, kc, vc, i32([[0, 1, 2], [3, -1, -1]]),
                                    i32([0, 0, 0]), i32([40, 9]), 0, 48, 0.125)
    torch.cuda.synchronize()
    assert unchanged(state, [kc, vc, k8, v8, k4, v4, ks, vs])


@pytest.mark.parametrize("algo,hq", [(pkv.PKV_ALGO_WAVE, 4), (pkv.PKV_ALGO_MFMA, 8)])
@pytest.mark.parametrize("parts", [0, 16, 512])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_a_batch_of_empty_contexts_gives_zero_rows(algo, hq, parts, out_dtype):
    """Every context 0 (max_context_len 0 too): nothing is attended, every
    row is zero, whatever the partition size and kernel."""
    rng = np.random.default_rng(71)
    nb, hkv, d, S = 4, 2, 128, 5
    kc = to_dev(np.full((nb, hkv, 16, d), np.nan, np.float32), "bf16")
    vc = kc.clone()
    q = to_dev(W.draw_normal(rng, (S, hq, d), "bf16"), "bf16")
    out = torch.full((S, hq, d), float("nan"), dtype=out_dtype, device=DEV)
    tables = i32(np.full((S, 1), -1))
    pkv.pkv_paged_attention_decode(out, q, kc, vc, tables, i32(np.zeros(S)), 0, 0.088, parts, algo)
    torch.cuda.synchronize()
    assert torch.equal(out.float().cpu(), torch.zeros((S, hq, d)))


@pytest.mark.parametrize("algo,hq,hkv,dtype", [
    (pkv.PKV_ALGO_WAVE, 8, 8, "bf16"), (pkv.PKV_ALGO_WAVE, 4, 4, "f32"),
    (pkv.PKV_ALGO_MFMA, 16, 2, "bf16"), (pkv.PKV_ALGO_MFMA, 8, 1, "f16")])
@pytest.mark.parametrize("parts", [0, 16, 48, 1024])
def test_contexts_that_fill_their_table_row(algo, hq, hkv, dtype, parts):
    """The longest context uses every entry of its table row (max_context_len
    = max_blocks x block_size); beside it a context one short of that, one
    just past a block edge, one of a single token.  Partitions of one tile
    (16 tokens: as many partitions as blocks), of three tiles (a ragged last
    partition) and of the whole row."""
    mb = 64
    full = mb * 16
    c = W.decode_case(72 + parts, 4, hq, hkv, 128, lens=[full, full - 1, 17, 1], dtype=dtype,
                      max_blocks=mb)
    assert c.block_tables.shape == (4, mb) and (c.block_tables[0] >= 0).all()
    dc = DevCase(c)
    got = out_f64(dc.decode(parts=parts, algo=algo, max_ctx=full))
    ref = A.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale)
    assert np.abs(got - ref).max() <= TOL
    # the one-token context is that token's value row, exactly
    one = c.block_tables[3, 0]
    for h in range(hq):
        np.testing.assert_array_equal(got[3, h], c.v_cache[one, h // (hq // hkv), 0].astype(np.float64))
