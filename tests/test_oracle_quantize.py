"""Pins of the int8 and 4-bit block encoders of the oracle
(oracle/quantize.py): hand-worked cases (tests/golden/int8_blocks.json,
int8_append.json, int4_blocks.json), the rounding error bound, sign
symmetry, exact power-of-two scaling, the unfilled-row rule, nibble packing
by brute force, and the bytes per token against the pages' figures
(kv_bytes.json, kv_compression.json)."""
import json
import os

import numpy as np
import pytest

from oracle import quantize as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int8_blocks.json")


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    x = np.asarray(case["rows"], np.float32)
    codes, s = Q.quantize_tile(x, case["filled"])
    assert codes.dtype == np.int8
    assert np.array_equal(codes, np.asarray(case["codes"], np.int8))
    assert s == np.float32(case["scale"])


def test_error_bound_and_range():
    rng = np.random.default_rng(0)
    for filled in (1, 7, 16):
        x = rng.standard_normal((16, 128)).astype(np.float32)
        codes, s = Q.quantize_tile(x, filled)
        rows = x[:filled].astype(np.float64)
        err = np.abs(codes[:filled].astype(np.float64) * float(s) - rows)
        # rint error is at most half a step; x / s carries one float32 rounding
        assert err.max() <= float(s) * (0.5 + 2.0 ** -16)
        assert np.abs(codes).max() == 127
        i = np.unravel_index(np.argmax(np.abs(rows)), rows.shape)
        assert abs(int(codes[:filled][i])) == 127
        assert not codes[filled:].any()


def test_sign_symmetry():
    x = np.random.default_rng(1).standard_normal((16, 64)).astype(np.float32)
    c1, s1 = Q.quantize_tile(x, 13)
    c2, s2 = Q.quantize_tile(-x, 13)
    assert s1 == s2 and np.array_equal(c1, -c2)


@pytest.mark.parametrize("k", [-3, 5])
def test_power_of_two_scaling_is_exact(k):
    x = np.random.default_rng(2).standard_normal((16, 32)).astype(np.float32)
    c1, s1 = Q.quantize_tile(x, 16)
    c2, s2 = Q.quantize_tile(x * np.float32(2.0 ** k), 16)
    assert np.array_equal(c1, c2) and s2 == s1 * np.float32(2.0 ** k)


def test_unfilled_rows_do_not_count():
    x = np.random.default_rng(3).standard_normal((16, 32)).astype(np.float32)
    y = x.copy()
    y[9:] = 1e6
    c1, s1 = Q.quantize_tile(x, 9)
    c2, s2 = Q.quantize_tile(y, 9)
    assert s1 == s2 and np.array_equal(c1, c2)


def test_quantize_blocks_touches_only_listed_blocks():
    rng = np.random.default_rng(4)
    pool = rng.standard_normal((6, 2, 16, 8)).astype(np.float32)
    codes = np.full(pool.shape, 55, np.int8)
    scales = np.full((6, 2), 9.0, np.float32)
    c2, s2 = Q.quantize_blocks(pool, codes, scales, [4, 1, 3], [16, 5, 0])
    for b in (0, 2, 3, 5):
        assert (c2[b] == 55).all() and (s2[b] == 9.0).all()
    for b, f in ((4, 16), (1, 5)):
        for h in range(2):
            c, s = Q.quantize_tile(pool[b, h], f)
            assert np.array_equal(c2[b, h], c) and s2[b, h] == s


# ------------------------------------------------------------ quantise-on-write
def _scale(text):
    num, _, den = text.partition("/")
    return np.float32(np.float32(float(num)) / np.float32(float(den))) if den else np.float32(float(num))


def test_append_hand_worked_cases():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "int8_append.json")))
    for case in g["cases"]:
        codes, s = np.zeros((4, 4), np.int8), np.float32(0)
        for st in case["steps"]:
            codes, s = Q.append_tile(codes, s, st["row0"], np.asarray(st["rows"], np.float32))
            want = np.asarray(st["codes"], np.int8)
            assert np.array_equal(codes[:len(want)], want), (case["name"], codes[:len(want)])
            assert s == _scale(st["scale"]), (case["name"], s)


def test_whole_block_write_is_the_block_encoder():
    rng = np.random.default_rng(31)
    for filled in (1, 7, 16):
        x = (rng.standard_normal((16, 64)) * 3).astype(np.float32)
        codes, s = Q.append_tile(np.full((16, 64), 99, np.int8), np.float32(5), 0, x[:filled])
        ref_codes, ref_s = Q.quantize_tile(x, filled)
        assert s == ref_s and np.array_equal(codes[:filled], ref_codes[:filled])


def test_appends_stay_within_the_rounding_bound():
    # token by token; each growth of the scale re-encodes the rows before it,
    # adding at most half a step of the new scale (plus float rounding)
    rng = np.random.default_rng(32)
    for trial in range(20):
        x = (rng.standard_normal((16, 32)) * rng.uniform(0.1, 10, (16, 1))).astype(np.float32)
        codes, s = np.zeros((16, 32), np.int8), np.float32(0)
        growths_after = np.zeros(16, np.int64)
        for r in range(16):
            s_prev = s
            codes, s = Q.append_tile(codes, s, r, x[r:r + 1])
            if r and s > s_prev:
                growths_after[:r] += 1
            assert s >= s_prev
            # every code stays in range and the scale covers the new row
            assert np.abs(codes).max() <= 127
            assert np.abs(x[r]).max() <= 127 * s * (1 + 1e-6)
        deq = codes.astype(np.float64) * np.float64(s)
        bound = (growths_after + 1)[:, None] * 0.5 * np.float64(s) * (1 + 1e-5)
        assert np.all(np.abs(deq - x) <= bound), trial


def test_runs_of_slot_mappings():
    assert list(Q.runs_of([5, 6, 7, 32, 33, -1, 8, 40], 16)) == [
        (0, 0, 5, 3), (3, 2, 0, 2), (6, 0, 8, 1), (7, 2, 8, 1)]
    # a run stops at a block edge and at a gap between rows
    assert list(Q.runs_of([14, 15, 16, 18], 16)) == [(0, 0, 14, 2), (2, 1, 0, 1), (3, 1, 2, 1)]
    assert list(Q.runs_of([], 16)) == []


def test_reshape_and_cache_int8_decode_step_matches_tile_appends():
    rng = np.random.default_rng(33)
    nb, h, d = 6, 2, 8
    kc = np.zeros((nb, h, 16, d), np.int8)
    vc = np.zeros_like(kc)
    ks = np.zeros((nb, h), np.float32)
    vs = np.zeros_like(ks)
    # two sequences: blocks 4 and 1, appended a token at a time
    for step in range(20):
        slots = [4 * 16 + step % 16 if step < 16 else 5 * 16 + step - 16, 1 * 16 + step % 16]
        key = rng.standard_normal((2, h, d)).astype(np.float32)
        val = rng.standard_normal((2, h, d)).astype(np.float32)
        nkc, nvc, nks, nvs = Q.reshape_and_cache_int8(key, val, kc, vc, ks, vs, slots, 16)
        for t, slot in enumerate(slots):
            b, r = slot // 16, slot % 16
            for hh in range(h):
                c, s = Q.append_tile(kc[b, hh], ks[b, hh], r, key[t:t + 1, hh])
                assert np.array_equal(nkc[b, hh], c) and nks[b, hh] == s
        kc, vc, ks, vs = nkc, nvc, nks, nvs


# ------------------------------------------------------------------ 4-bit
GOLDEN4 = os.path.join(os.path.dirname(__file__), "golden", "int4_blocks.json")


@pytest.mark.parametrize("case", json.load(open(GOLDEN4))["cases"], ids=lambda c: c["name"])
def test_int4_hand_worked_cases(case):
    codes, s = Q.quantize_tile(np.asarray(case["rows"], np.float32), case["filled"], Q.INT4_MAX)
    assert np.array_equal(codes, np.asarray(case["codes"], np.int8))
    assert s == _scale(case["scale"])
    assert np.array_equal(Q.pack_int4(codes), np.asarray(case["bytes"], np.uint8))


def test_int4_append_hand_worked_cases():
    for case in json.load(open(GOLDEN4))["append"]:
        codes, s = np.zeros((4, 4), np.int8), np.float32(0)
        for st in case["steps"]:
            codes, s = Q.append_tile(codes, s, st["row0"], np.asarray(st["rows"], np.float32),
                                     Q.INT4_MAX)
            want = np.asarray(st["codes"], np.int8)
            assert np.array_equal(codes[:len(want)], want), (case["name"], codes[:len(want)])
            assert s == _scale(st["scale"]), (case["name"], s)


def test_int4_nibble_packing_brute_force():
    # every code pair: the byte is (hi & 15) << 4 | (lo & 15), and unpacking inverts it
    lo, hi = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8), indexing="ij")
    pairs = np.stack([lo.ravel(), hi.ravel()], 1).astype(np.int8)
    b = Q.pack_int4(pairs)[:, 0]
    assert sorted(b.tolist()) == list(range(256))
    for (x, y), byte in zip(pairs.tolist(), b.tolist()):
        assert byte == ((y & 15) << 4) | (x & 15)
    assert np.array_equal(Q.unpack_int4(b[:, None]), pairs)
    with pytest.raises(ValueError):
        Q.pack_int4(np.array([8, 0]))
    with pytest.raises(ValueError):
        Q.pack_int4(np.array([1, 2, 3]))


def test_int4_error_bound_and_range():
    rng = np.random.default_rng(40)
    for filled in (1, 7, 16):
        x = rng.standard_normal((16, 128)).astype(np.float32)
        codes, s = Q.quantize_tile(x, filled, Q.INT4_MAX)
        rows = x[:filled].astype(np.float64)
        err = np.abs(codes[:filled].astype(np.float64) * float(s) - rows)
        assert err.max() <= float(s) * (0.5 + 2.0 ** -16)
        assert np.abs(codes).max() == 7
        i = np.unravel_index(np.argmax(np.abs(rows)), rows.shape)
        assert abs(int(codes[:filled][i])) == 7
        assert not codes[filled:].any()
        # sixteen times coarser than int8 on the same tile
        c8, s8 = Q.quantize_tile(x, filled)
        assert s == np.float32(np.float32(np.abs(rows).max()) / np.float32(7))
        assert s8 == np.float32(np.float32(np.abs(rows).max()) / np.float32(127))


def test_int4_sign_symmetry_and_power_of_two_scaling():
    x = np.random.default_rng(41).standard_normal((16, 64)).astype(np.float32)
    c1, s1 = Q.quantize_tile(x, 13, Q.INT4_MAX)
    c2, s2 = Q.quantize_tile(-x, 13, Q.INT4_MAX)
    assert s1 == s2 and np.array_equal(c1, -c2)
    c3, s3 = Q.quantize_tile(x * np.float32(8), 13, Q.INT4_MAX)
    assert np.array_equal(c1, c3) and s3 == s1 * np.float32(8)


def test_int4_blocks_round_trip_through_packing():
    rng = np.random.default_rng(42)
    pool = rng.standard_normal((5, 2, 16, 8)).astype(np.float32)
    packed = np.full((5, 2, 16, 4), 0x5A, np.uint8)
    scales = np.full((5, 2), 3.0, np.float32)
    p2, s2 = Q.quantize_blocks_int4(pool, packed, scales, [3, 0], [16, 9])
    for b in (1, 2, 4):
        assert (p2[b] == 0x5A).all() and (s2[b] == 3.0).all()
    for b, f in ((3, 16), (0, 9)):
        for h in range(2):
            c, s = Q.quantize_tile(pool[b, h], f, Q.INT4_MAX)
            assert np.array_equal(Q.unpack_int4(p2[b, h]), c) and s2[b, h] == s


def test_int4_appends_stay_within_the_rounding_bound():
    rng = np.random.default_rng(43)
    for trial in range(20):
        x = (rng.standard_normal((16, 32)) * rng.uniform(0.1, 10, (16, 1))).astype(np.float32)
        codes, s = np.zeros((16, 32), np.int8), np.float32(0)
        growths_after = np.zeros(16, np.int64)
        for r in range(16):
            s_prev = s
            codes, s = Q.append_tile(codes, s, r, x[r:r + 1], Q.INT4_MAX)
            if r and s > s_prev:
                growths_after[:r] += 1
            assert np.abs(codes).max() <= 7
        deq = codes.astype(np.float64) * np.float64(s)
        bound = (growths_after + 1)[:, None] * 0.5 * np.float64(s) * (1 + 1e-5)
        assert np.all(np.abs(deq - x) <= bound), trial


def test_reshape_and_cache_int4_is_the_int8_write_on_4bit_codes():
    rng = np.random.default_rng(44)
    nb, h, d = 4, 2, 8
    kp = np.zeros((nb, h, 16, d // 2), np.uint8)
    vp = np.zeros_like(kp)
    ks = np.zeros((nb, h), np.float32)
    vs = np.zeros_like(ks)
    for step in range(18):
        slots = [2 * 16 + step if step < 16 else 3 * 16 + step - 16]
        key = (rng.standard_normal((1, h, d)) * (1 + step)).astype(np.float32)
        val = rng.standard_normal((1, h, d)).astype(np.float32)
        nkp, nvp, nks, nvs = Q.reshape_and_cache_int4(key, val, kp, vp, ks, vs, slots, 16)
        b, r = slots[0] // 16, slots[0] % 16
        for hh in range(h):
            c, s = Q.append_tile(Q.unpack_int4(kp[b, hh]), ks[b, hh], r, key[:, hh], Q.INT4_MAX)
            assert np.array_equal(Q.unpack_int4(nkp[b, hh]), c) and nks[b, hh] == s
        kp, vp, ks, vs = nkp, nvp, nks, nvs


def test_kv_bytes_against_the_pages():
    # one token of LLaMA-7B at fp16 (kongchang.com worked figure) and the
    # cnnetsun.cn compression table's memory column against fp32
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_bytes.json")))
    assert Q.kv_bytes_per_token(g["layers"], g["heads"], g["head_dim"], 8 * g["elem_bytes"]) == \
        g["kv_bytes_per_token_all_layers"]
    assert Q.kv_bytes_per_token(1, g["heads"], g["head_dim"], 16) == g["kv_bytes_per_token_one_layer"]
    t = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_compression.json")))
    full = Q.kv_bytes_per_token(32, 32, 128, 32)
    for row in t["rows"]:
        assert 1 - Q.kv_bytes_per_token(32, 32, 128, row["bits"]) / full == row["reduction"], row
