"""Pins of the int8 block encoder of the oracle (oracle/quantize.py):
hand-worked cases (tests/golden/int8_blocks.json), the rounding error bound,
sign symmetry, exact power-of-two scaling, and the unfilled-row rule."""
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
