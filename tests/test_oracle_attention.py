"""Pins of the attention oracle against things other than itself.

Library routines (torch's CPU scaled_dot_product_attention in float64,
scipy's softmax), brute force with ``math.exp`` over never-paged K/V, closed
forms and invariants.  Each catches a different plausible slip: a wrong block
or row index in the gather, a dropped scale, a transposed operand, an
unmasked tail, a wrong causal offset, a wrong head grouping.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as A
from synth import workloads as W


def sdpa64(q, K, V, scale, mask=None):
    """torch SDPA on CPU in float64. q [Lq, D], K/V [n, D]."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None]
    kt = torch.from_numpy(np.asarray(K, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(V, np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                         scale=float(scale))
    return o[0, 0].numpy()


@pytest.fixture(scope="module")
def tiny():
    return W.tiny_decode(seed=0, keep_logical=True)


def test_gather_is_bit_identical_to_never_paged_rows(tiny):
    for s, n in enumerate(tiny.context_lens):
        K = A.gather(tiny.k_cache, tiny.block_tables[s], n, 16)
        V = A.gather(tiny.v_cache, tiny.block_tables[s], n, 16)
        assert np.array_equal(K, tiny.k_logical[s].astype(np.float64))
        assert np.array_equal(V, tiny.v_logical[s].astype(np.float64))


def test_decode_matches_torch_sdpa_on_unpaged_kv(tiny):
    out = A.decode(tiny.q, tiny.k_cache, tiny.v_cache, tiny.block_tables,
                   tiny.context_lens, tiny.scale)
    for s in range(4):
        for h in range(8):
            ref = sdpa64(tiny.q[s, h][None], tiny.k_logical[s][:, h], tiny.v_logical[s][:, h],
                         tiny.scale)[0]
            np.testing.assert_allclose(out[s, h], ref, rtol=0, atol=1e-12)


def test_decode_matches_brute_force_loops():
    c = W.decode_case(7, 2, 2, 2, 4, lens=[1, 19], dtype="f32", num_blocks=6,
                      keep_logical=True)
    out = A.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale)
    for s in range(2):
        n = int(c.context_lens[s])
        for h in range(2):
            xs = []
            for t in range(n):
                dot = 0.0
                for d in range(4):
                    dot += float(c.q[s, h, d]) * float(c.k_logical[s][t, h, d])
                xs.append(float(c.scale) * dot)
            mx = max(xs)
            es = [math.exp(x - mx) for x in xs]
            z = sum(es)
            for d in range(4):
                o = sum(es[t] / z * float(c.v_logical[s][t, h, d]) for t in range(n))
                assert abs(out[s, h, d] - o) < 1e-13


def test_weights_match_scipy_and_sum_to_one(tiny):
    for s in range(4):
        for h in (0, 7):
            w = A.decode_weights(tiny.q, tiny.k_cache, tiny.block_tables, tiny.context_lens,
                                 tiny.scale, s, h)
            x = np.float64(tiny.scale) * (tiny.k_logical[s][:, h].astype(np.float64)
                                          @ tiny.q[s, h].astype(np.float64))
            np.testing.assert_allclose(w, scipy.special.softmax(x), rtol=0, atol=1e-15)
            assert abs(w.sum() - 1.0) <= 1e-12


def test_zero_query_and_zero_scale_give_mean_of_values(tiny):
    q0 = np.zeros_like(tiny.q)
    out = A.decode(q0, tiny.k_cache, tiny.v_cache, tiny.block_tables, tiny.context_lens,
                   tiny.scale)
    out2 = A.decode(tiny.q, tiny.k_cache, tiny.v_cache, tiny.block_tables,
                    tiny.context_lens, np.float32(0))
    for s in range(4):
        mean = tiny.v_logical[s].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(out[s], mean, rtol=0, atol=1e-14)
        np.testing.assert_allclose(out2[s], mean, rtol=0, atol=1e-14)


def test_equal_keys_give_uniform_weights():
    c = W.decode_case(3, 1, 2, 2, 8, lens=[37], dtype="f32", num_blocks=5, keep_logical=True)
    row = c.k_logical[0][5]
    kc = c.k_cache.copy()
    for t in range(37):
        kc[c.block_tables[0][t // 16], :, t % 16, :] = row
    out = A.decode(c.q, kc, c.v_cache, c.block_tables, c.context_lens, c.scale)
    np.testing.assert_allclose(out[0], c.v_logical[0].astype(np.float64).mean(0),
                               rtol=0, atol=1e-14)


def test_context_one_returns_first_value_row_exactly(tiny):
    lens = np.ones(4, np.int32)
    out = A.decode(tiny.q, tiny.k_cache, tiny.v_cache, tiny.block_tables, lens, tiny.scale)
    for s in range(4):
        assert np.array_equal(out[s], tiny.v_logical[s][0].astype(np.float64))


def test_context_zero_gives_zero_row(tiny):
    lens = tiny.context_lens.copy()
    lens[2] = 0
    out = A.decode(tiny.q, tiny.k_cache, tiny.v_cache, tiny.block_tables, lens, tiny.scale)
    assert np.all(out[2] == 0)


def test_table_entry_outside_the_pool_is_rejected(tiny):
    bad = tiny.block_tables.copy()
    bad[1, 2] = -1
    with pytest.raises(ValueError):
        A.decode(tiny.q, tiny.k_cache, tiny.v_cache, bad, tiny.context_lens, tiny.scale)


def test_two_tokens_match_logistic_closed_form():
    c = W.decode_case(11, 1, 1, 1, 16, lens=[2], dtype="f32", num_blocks=1, keep_logical=True)
    K = c.k_logical[0][:, 0].astype(np.float64)
    V = c.v_logical[0][:, 0].astype(np.float64)
    q = c.q[0, 0].astype(np.float64)
    x0, x1 = np.float64(c.scale) * (K @ q)
    w0 = 1.0 / (1.0 + math.exp(x1 - x0))
    out = A.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale)
    np.testing.assert_allclose(out[0, 0], w0 * V[0] + (1 - w0) * V[1], rtol=0, atol=1e-14)


def test_large_scores_select_the_argmax_row(tiny):
    q = tiny.q * np.float32(100)
    out = A.decode(q, tiny.k_cache, tiny.v_cache, tiny.block_tables, tiny.context_lens,
                   tiny.scale)
    checked = 0
    for s in range(4):
        for h in range(8):
            x = tiny.k_logical[s][:, h].astype(np.float64) @ q[s, h].astype(np.float64)
            top = np.sort(x)[-2:]
            if float(tiny.scale) * (top[1] - top[0]) < 40.0:  # no clear winner
                continue
            checked += 1
            np.testing.assert_allclose(out[s, h], tiny.v_logical[s][np.argmax(x), h],
                                       rtol=0, atol=1e-12)
    assert checked >= 8


def test_physical_placement_does_not_change_output(tiny):
    base = A.decode(tiny.q, tiny.k_cache, tiny.v_cache, tiny.block_tables, tiny.context_lens,
                    tiny.scale)
    rng = np.random.default_rng(5)
    perm = rng.permutation(tiny.num_blocks)          # physical block b -> perm[b]
    kc = np.empty_like(tiny.k_cache)
    vc = np.empty_like(tiny.v_cache)
    kc[perm] = tiny.k_cache
    vc[perm] = tiny.v_cache
    tables = np.where(tiny.block_tables >= 0, perm[np.maximum(tiny.block_tables, 0)], -1)
    out = A.decode(tiny.q, kc, vc, tables.astype(np.int32), tiny.context_lens, tiny.scale)
    assert np.array_equal(out, base)


@pytest.mark.parametrize("bs", [1, 8, 32])
def test_block_size_does_not_change_output(tiny, bs):
    base = A.decode(tiny.q, tiny.k_cache, tiny.v_cache, tiny.block_tables, tiny.context_lens,
                    tiny.scale)
    nbs = [W.blocks_for(n, bs) for n in tiny.context_lens]
    perm = np.random.default_rng(9).permutation(sum(nbs) + 3).astype(np.int32)
    tables = W.place_by_permutation(tiny.context_lens, perm, bs)
    kc = np.full((len(perm), 8, bs, 64), np.nan, np.float32)
    vc = np.full_like(kc, np.nan)
    for s in range(4):
        W.scatter_rows(kc, tables[s], tiny.k_logical[s], bs)
        W.scatter_rows(vc, tables[s], tiny.v_logical[s], bs)
    out = A.decode(tiny.q, kc, vc, tables, tiny.context_lens, tiny.scale, block_size=bs)
    assert np.array_equal(out, base)


def test_key_order_does_not_change_output(tiny):
    base = A.decode(tiny.q, tiny.k_cache, tiny.v_cache, tiny.block_tables, tiny.context_lens,
                    tiny.scale)
    rng = np.random.default_rng(13)
    kc = tiny.k_cache.copy()
    vc = tiny.v_cache.copy()
    for s, n in enumerate(tiny.context_lens):
        order = rng.permutation(int(n))
        W.scatter_rows(kc, tiny.block_tables[s], tiny.k_logical[s][order], 16)
        W.scatter_rows(vc, tiny.block_tables[s], tiny.v_logical[s][order], 16)
    out = A.decode(tiny.q, kc, vc, tiny.block_tables, tiny.context_lens, tiny.scale)
    np.testing.assert_allclose(out, base, rtol=0, atol=1e-13)


def test_grouped_heads_equal_mha_with_repeated_kv():
    c = W.decode_case(21, 3, 8, 2, 32, lens=[5, 33, 64], dtype="bf16", keep_logical=True)
    out = A.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale)
    kc = np.repeat(c.k_cache, 4, axis=1)
    vc = np.repeat(c.v_cache, 4, axis=1)
    out_mha = A.decode(c.q, kc, vc, c.block_tables, c.context_lens, c.scale)
    assert np.array_equal(out, out_mha)
    # and against SDPA with explicitly repeated heads
    for s in range(3):
        for h in range(8):
            ref = sdpa64(c.q[s, h][None], c.k_logical[s][:, h // 4], c.v_logical[s][:, h // 4],
                         c.scale)[0]
            np.testing.assert_allclose(out[s, h], ref, rtol=0, atol=1e-12)


def test_int8_storage_with_unit_scale_equals_float_path():
    c = W.decode_case(31, 2, 4, 2, 16, lens=[9, 40], dtype="f32", keep_logical=False)
    rng = np.random.default_rng(2)
    codes = rng.integers(-127, 128, size=c.k_cache.shape).astype(np.int8)
    vcodes = rng.integers(-127, 128, size=c.v_cache.shape).astype(np.int8)
    ones = np.ones((c.num_blocks, c.kv_heads), np.float32)
    out_i8 = A.decode(c.q, codes, vcodes, c.block_tables, c.context_lens, c.scale,
                      k_scale=ones, v_scale=ones)
    out_f = A.decode(c.q, codes.astype(np.float32), vcodes.astype(np.float32), c.block_tables,
                     c.context_lens, c.scale)
    assert np.array_equal(out_i8, out_f)


def test_int8_gather_decodes_within_half_a_step():
    c = W.decode_case(41, 3, 4, 2, 32, lens=[3, 16, 45], dtype="bf16", int8=True,
                      keep_logical=True)
    for s, n in enumerate(c.context_lens):
        K = A.gather(c.k_i8, c.block_tables[s], n, 16, c.k_scale)
        blocks = c.block_tables[s][np.arange(n) // 16]
        half = c.k_scale[blocks].astype(np.float64)[:, :, None] / 2
        err = np.abs(K - c.k_logical[s].astype(np.float64))
        # half a quantisation step, plus the fp32 rounding of x / s before rint
        assert np.all(err <= half * (1 + 1e-5))
        # the largest |x| of each tile decodes exactly to +-127 * scale
        assert np.all(np.abs(c.k_i8[blocks[0], :, 0, :]).max(axis=-1) <= 127)


@pytest.fixture(scope="module")
def chunks():
    return W.prefill_case(17, 4, 2, 32, [(0, 20), (7, 9), (33, 1), (16, 16)], dtype="bf16",
                          keep_logical=True)


def test_prefill_matches_sdpa_with_bottom_right_causal_mask(chunks):
    c = chunks
    out = A.prefill(c.q, c.k_cache, c.v_cache, c.block_tables, c.query_start_loc,
                    c.context_lens, c.scale)
    for s in range(len(c.context_lens)):
        a, b = c.query_start_loc[s], c.query_start_loc[s + 1]
        n = int(c.context_lens[s])
        qlen = b - a
        mask = np.arange(n)[None, :] <= (n - qlen + np.arange(qlen))[:, None]
        for h in range(4):
            ref = sdpa64(c.q[a:b, h], c.k_logical[s][:, h // 2], c.v_logical[s][:, h // 2],
                         c.scale, mask=mask)
            np.testing.assert_allclose(out[a:b, h], ref, rtol=0, atol=1e-12)


def test_prefill_row_equals_decode_over_truncated_context(chunks):
    c = chunks
    out = A.prefill(c.q, c.k_cache, c.v_cache, c.block_tables, c.query_start_loc,
                    c.context_lens, c.scale)
    for s in range(len(c.context_lens)):
        a, b = int(c.query_start_loc[s]), int(c.query_start_loc[s + 1])
        n = int(c.context_lens[s])
        for i in range(b - a):
            lens = np.array([n - (b - a) + i + 1], np.int32)
            d = A.decode(c.q[a + i][None], c.k_cache, c.v_cache, c.block_tables[s][None], lens,
                         c.scale)
            assert np.array_equal(out[a + i], d[0])


def test_prefill_of_one_row_is_decode(tiny):
    qsl = np.arange(5, dtype=np.int32)
    out = A.prefill(tiny.q, tiny.k_cache, tiny.v_cache, tiny.block_tables, qsl,
                    tiny.context_lens, tiny.scale)
    d = A.decode(tiny.q, tiny.k_cache, tiny.v_cache, tiny.block_tables, tiny.context_lens,
                 tiny.scale)
    assert np.array_equal(out, d)
