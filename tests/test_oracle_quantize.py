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
