"""Cache writes and block copies, as their plain definitions.

* ``reshape_and_cache``: only the new token's K/V is computed and appended to
  the cache each step ([nxbn] section 一); the per-token physical address is
  recorded by the page table ([nxbn] §2.2).  Here row t of the new keys and
  values goes to block ``slot // block_size``, row ``slot % block_size``, for
  every head; a negative slot means "skip this row".
* ``copy_blocks``: the data copy of copy-on-write — a new block receives the
  contents of the shared one before the writer appends ([kongchang] section
  "KV Cache内存共享").  Each (src, dst) pair copies K, V and, for int8
  storage, the per-block scales.

Both return new arrays and leave the inputs untouched.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np


def reshape_and_cache(key: np.ndarray, value: np.ndarray, k_cache: np.ndarray,
                      v_cache: np.ndarray, slot_mapping: Sequence[int],
                      block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    kc = k_cache.copy()
    vc = v_cache.copy()
    for t, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        kc[slot // block_size, :, slot % block_size, :] = key[t]
        vc[slot // block_size, :, slot % block_size, :] = value[t]
    return kc, vc


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs: Sequence[Tuple[int, int]],
                k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None):
    kc = k_cache.copy()
    vc = v_cache.copy()
    ks = None if k_scale is None else k_scale.copy()
    vs = None if v_scale is None else v_scale.copy()
    for src, dst in pairs:
        kc[int(dst)] = k_cache[int(src)]
        vc[int(dst)] = v_cache[int(src)]
        if ks is not None:
            ks[int(dst)] = k_scale[int(src)]
        if vs is not None:
            vs[int(dst)] = v_scale[int(src)]
    return kc, vc, ks, vs
