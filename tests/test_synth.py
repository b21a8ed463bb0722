"""The input generators: rounding matches torch's conversions, draws are
reproducible, and the pool layout puts every row where the table says."""
import numpy as np
import torch

from synth import workloads as W


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.00390625, 1.01171875]   # ties
    ours = W.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    bits = W.storage_array(ours, "bf16")
    assert np.array_equal(W.from_bf16_bits(bits), ours)


def test_f16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float16).to(torch.float32).numpy()
    assert np.array_equal(W.round_to(x, "f16"), ref)


def test_cases_are_reproducible_and_placed_by_table():
    a = W.decode_case(5, 3, 4, 2, 16, len_range=(1, 40), keep_logical=True)
    b = W.decode_case(5, 3, 4, 2, 16, len_range=(1, 40), keep_logical=True)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.k_cache.view(np.uint32), b.k_cache.view(np.uint32))
    owned = set()
    for s, n in enumerate(a.context_lens):
        for p in range(n):
            blk = a.block_tables[s][p // 16]
            owned.add((int(blk), p % 16))
            assert np.array_equal(a.k_cache[blk, :, p % 16, :], a.k_logical[s][p])
    for blk in range(a.num_blocks):
        for r in range(16):
            if (blk, r) not in owned:
                assert np.all(np.isnan(a.k_cache[blk, :, r, :]))


def test_quantiser_extremes():
    x = np.array([[0.5, -2.0], [1.0, 0.25]], np.float32)
    q, s = W.quantize_int8(x)
    assert s == np.float32(2.0) / np.float32(127.0)
    assert q[0, 1] == -127 and np.abs(q).max() == 127
    q0, s0 = W.quantize_int8(np.zeros((3, 2), np.float32))
    assert s0 == 0 and not q0.any()


def test_prefix_sharing_rows_follow_tokens():
    c = W.prefix_sharing(seed=3, num_requests=5, system_len=40, own_lens=(1, 20),
                         shared_lens=[40, 40, 17, 0, 33], q_heads=4, kv_heads=2, head_dim=16)
    for r in range(5):
        for s in range(5):
            a, b = c.prompts[r], c.prompts[s]
            m = min(len(a), len(b))
            same = int(np.argmin(a[:m] == b[:m])) if not np.array_equal(a[:m], b[:m]) else m
            # rows agree exactly where the token prefixes agree, and only there
            assert np.array_equal(c.k[r][:same], c.k[s][:same])
            assert np.array_equal(c.v[r][:same], c.v[s][:same])
            if r != s and same < m:
                assert not np.array_equal(c.k[r][same], c.k[s][same])
            if r != s:
                assert same == min(c.shared_lens[r], c.shared_lens[s])
