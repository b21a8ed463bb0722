"""Int8 storage of whole KV blocks, as its definition — TEST INFRASTRUCTURE ONLY.

The cnnetsun.cn page ("别再让GPU内存拖后腿了…") lists INT8 KV in its memory
compression table (§3.2 内存压缩技术: a quarter of fp32's bytes) and, for
long documents, turns INT8 on for the historical pages (§4.3
典型场景优化策略).  The encoding itself is not on the pages.  Reading taken
here: symmetric codes per (block, KV head), over the block's filled rows,

    a     = max |x|                          (float32)
    s     = float32(a / 127)                 (IEEE division, nearest even)
    code  = 0                                   if s == 0
          = clip(rint(float32(x / s)), -127, 127) otherwise
                                             (IEEE division; rint ties to even)

and rows past the filled count get code 0.  A scale below the smallest
normal float32 (a block whose values are all below about 1.5e-36) counts as
zero: such a block stores all-zero codes.

Everything is float32 arithmetic, as the definition states: the result is
unique bit for bit.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

SMALLEST_NORMAL = np.float32(np.finfo(np.float32).tiny)


def quantize_tile(x: np.ndarray, filled: int) -> Tuple[np.ndarray, np.float32]:
    """Codes ``int8 [rows, D]`` and the scale of one (block, KV head) tile
    whose first ``filled`` rows hold data."""
    x = np.asarray(x, dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.int8)
    filled = int(filled)
    if filled <= 0:
        return codes, np.float32(0)
    rows = x[:filled]
    a = np.float32(np.max(np.abs(rows)))
    s = np.float32(a / np.float32(127))
    if s < SMALLEST_NORMAL:
        return codes, np.float32(0)
    q = np.rint((rows / s).astype(np.float32))
    codes[:filled] = np.clip(q, -127, 127).astype(np.int8)
    return codes, s


def quantize_blocks(pool: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                    blocks: Sequence[int], filled: Sequence[int]):
    """Encode the listed blocks of a float pool ``[NB, H, BS, D]`` (values
    exactly as stored) into copies of an int8 pool and its ``[NB, H]``
    scales; blocks not listed keep what they held.  A filled count of 0
    leaves the block untouched."""
    out_codes = np.array(codes, dtype=np.int8, copy=True)
    out_scales = np.array(scales, dtype=np.float32, copy=True)
    for b, f in zip(blocks, filled):
        b, f = int(b), int(f)
        if f <= 0:
            continue
        for h in range(pool.shape[1]):
            out_codes[b, h], out_scales[b, h] = quantize_tile(pool[b, h], f)
    return out_codes, out_scales
